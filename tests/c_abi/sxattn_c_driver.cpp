// A plain host program that drives libsxattn through its C ABI alone (no Python,
// no PyTorch): HIP device buffers, the library's calls, and files in and out.
//
// Usage: sxattn_c_driver DIR
// DIR/args.txt holds: n_blk hq hkv d n_ctx chunk_size n_bin n_chunk
// DIR/{anchor,start}.bin   int32 [n_blk]
// DIR/{gs,gl}.bin          int32 [n_chunk]: the local chunk list (global start, length)
// DIR/{q,ks,vs}.bin        bf16 bits [16 n_blk][hq | hkv][d]
// DIR/{k,v}.bin            bf16 bits [sum gl][hkv][d]: the listed chunks back to back
// DIR/dout.bin             bf16 bits [16 n_blk][hq][d]
// DIR/{ggs,ggl}.bin        int32 [2]: two row ranges of k for the gather
// Writes:
// DIR/cost.bin   int64 [ceil(n_ctx / chunk_size)]   chunk_cost over the whole context
// DIR/bins.bin   int32, DIR/load.bin int64          lpt_assign of those costs onto n_bin
// DIR/dbins.bin, dload.bin, dplan_gs.bin, dplan_gl.bin  lpt_plan of the device costs (its
//                bins and loads, and each bin's chunk starts and lengths [n_bin][n_all / n_bin])
// DIR/o.bin      bf16 bits, DIR/lse.bin float32     sparse_xattn_fwd over every listed chunk
//                                                   plus the own-block term
// DIR/o2.bin, DIR/lse2.bin                          the same from two calls (first half of the
//                                                   chunks with the own-block term, then the
//                                                   rest) merged by lse_combine
// DIR/kg.bin     bf16 bits                          context_gather of the two k row ranges
// DIR/{dq,dk,dv,dks,dvs}.bin float32                 sparse_xattn_bwd (all phases, dq
//                                                   overwritten, load-balanced) from o, lse
// Exit status 0 on success; on a library error it prints sxa_last_error().
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <fstream>
#include <stdexcept>
#include <string>
#include <vector>

#include "sxattn.h"

namespace {

template <typename T>
std::vector<T> read_file(const std::string& path, size_t n) {
  std::vector<T> v(n);
  std::ifstream f(path, std::ios::binary);
  if (!f || !f.read(reinterpret_cast<char*>(v.data()), static_cast<std::streamsize>(n * sizeof(T))))
    throw std::runtime_error("cannot read " + path);
  return v;
}

template <typename T>
void write_file(const std::string& path, const std::vector<T>& v) {
  std::ofstream f(path, std::ios::binary);
  f.write(reinterpret_cast<const char*>(v.data()), static_cast<std::streamsize>(v.size() * sizeof(T)));
  if (!f) throw std::runtime_error("cannot write " + path);
}

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) throw std::runtime_error(std::string(what) + ": " + hipGetErrorString(e));
}

void sxa_check(int st, const char* what) {
  if (st != SXA_OK) throw std::runtime_error(std::string(what) + ": " + sxa_last_error());
}

// a device copy of a host vector, freed with the object
template <typename T>
struct Dev {
  T* p = nullptr;
  size_t n = 0;
  explicit Dev(size_t count) : n(count) { hip_check(hipMalloc(&p, std::max<size_t>(count, 1) * sizeof(T)), "hipMalloc"); }
  explicit Dev(const std::vector<T>& h) : Dev(h.size()) {
    hip_check(hipMemcpy(p, h.data(), n * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy H2D");
  }
  std::vector<T> host() const {
    std::vector<T> h(n);
    hip_check(hipMemcpy(h.data(), p, n * sizeof(T), hipMemcpyDeviceToHost), "hipMemcpy D2H");
    return h;
  }
  ~Dev() { hipFree(p); }
  Dev(const Dev&) = delete;
  Dev& operator=(const Dev&) = delete;
};

int run(const std::string& dir) {
  int64_t n_blk, hq, hkv, d, n_ctx, chunk_size, n_bin, n_chunk;
  {
    std::ifstream a(dir + "/args.txt");
    if (!(a >> n_blk >> hq >> hkv >> d >> n_ctx >> chunk_size >> n_bin >> n_chunk))
      throw std::runtime_error("cannot read args.txt");
  }
  const int64_t n_q = 16 * n_blk;
  const auto anchor = read_file<int32_t>(dir + "/anchor.bin", n_blk);
  const auto start = read_file<int32_t>(dir + "/start.bin", n_blk);
  const auto gs = read_file<int32_t>(dir + "/gs.bin", n_chunk);
  const auto gl = read_file<int32_t>(dir + "/gl.bin", n_chunk);
  int64_t n_loc = 0;
  for (int32_t len : gl) n_loc += len;
  const auto q = read_file<uint16_t>(dir + "/q.bin", n_q * hq * d);
  const auto ks = read_file<uint16_t>(dir + "/ks.bin", n_q * hkv * d);
  const auto vs = read_file<uint16_t>(dir + "/vs.bin", n_q * hkv * d);
  const auto k = read_file<uint16_t>(dir + "/k.bin", n_loc * hkv * d);
  const auto v = read_file<uint16_t>(dir + "/v.bin", n_loc * hkv * d);
  const auto dout = read_file<uint16_t>(dir + "/dout.bin", n_q * hq * d);
  const auto ggs = read_file<int32_t>(dir + "/ggs.bin", 2);
  const auto ggl = read_file<int32_t>(dir + "/ggl.bin", 2);

  Dev<int32_t> d_anchor(anchor), d_start(start), d_gs(gs), d_gl(gl);
  Dev<uint16_t> d_q(q), d_ks(ks), d_vs(vs), d_k(k), d_v(v);
  hipStream_t s;
  hip_check(hipStreamCreate(&s), "hipStreamCreate");

  // chunk costs over the whole context, then the LPT plan on the host
  const int64_t n_all = (n_ctx + chunk_size - 1) / chunk_size;
  Dev<int64_t> d_cost(n_all);
  sxa_check(chunk_cost(d_anchor.p, d_start.p, static_cast<int32_t>(n_blk), 16, static_cast<int32_t>(n_ctx),
                       static_cast<int32_t>(chunk_size), d_cost.p, s),
            "chunk_cost");
  hip_check(hipStreamSynchronize(s), "sync");
  const auto cost = d_cost.host();
  std::vector<int32_t> bins(n_all);
  std::vector<int64_t> load(n_bin);
  sxa_check(lpt_assign(cost.data(), static_cast<int32_t>(n_all), static_cast<int32_t>(n_bin), bins.data(),
                       load.data()),
            "lpt_assign");
  write_file(dir + "/cost.bin", cost);
  write_file(dir + "/bins.bin", bins);
  write_file(dir + "/load.bin", load);
  // the same plan on the device, from the device costs, with each bin's chunk list
  std::vector<int32_t> all_gs(n_all), all_gl(n_all);
  for (int64_t c = 0; c < n_all; ++c) {
    all_gs[c] = static_cast<int32_t>(c * chunk_size);
    all_gl[c] = static_cast<int32_t>(std::min<int64_t>(chunk_size, n_ctx - c * chunk_size));
  }
  Dev<int32_t> d_all_gs(all_gs), d_all_gl(all_gl), d_bins(n_all), d_plan_gs(n_all), d_plan_gl(n_all);
  Dev<int64_t> d_load(n_bin);
  sxa_check(lpt_plan(d_cost.p, d_all_gs.p, d_all_gl.p, static_cast<int32_t>(n_all), static_cast<int32_t>(n_bin),
                     d_bins.p, d_load.p, d_plan_gs.p, d_plan_gl.p, s),
            "lpt_plan");
  hip_check(hipStreamSynchronize(s), "sync");
  write_file(dir + "/dbins.bin", d_bins.host());
  write_file(dir + "/dload.bin", d_load.host());
  write_file(dir + "/dplan_gs.bin", d_plan_gs.host());
  write_file(dir + "/dplan_gl.bin", d_plan_gl.host());

  // forward over every listed chunk, with the own-block term
  const int64_t rows = n_q * hq;
  std::vector<uint8_t> ws_h(static_cast<size_t>(sparse_xattn_fwd_workspace_bytes(
      static_cast<int32_t>(n_blk), static_cast<int32_t>(hq), static_cast<int32_t>(hkv))));
  Dev<uint8_t> d_ws(ws_h.size());
  Dev<uint16_t> d_o(rows * d);
  Dev<float> d_lse(rows);
  sxa_check(sparse_xattn_fwd(d_q.p, d_k.p, d_v.p, SXA_BF16, static_cast<int32_t>(n_blk), 16,
                             static_cast<int32_t>(hq), static_cast<int32_t>(hkv), static_cast<int32_t>(d),
                             static_cast<float>(1.0 / std::sqrt(static_cast<double>(d))), d_anchor.p,
                             d_start.p, d_gs.p, d_gl.p, static_cast<int32_t>(n_chunk), n_loc, d_ks.p, d_vs.p,
                             d_o.p, SXA_BF16, d_lse.p, d_ws.p, static_cast<int64_t>(ws_h.size()), s),
            "sparse_xattn_fwd");
  hip_check(hipStreamSynchronize(s), "sync");
  write_file(dir + "/o.bin", d_o.host());
  write_file(dir + "/lse.bin", d_lse.host());

  // two calls over the two halves of the chunk list (float32 partials), then the combine
  const int64_t c1 = n_chunk / 2;
  int64_t loc1 = 0;
  for (int64_t c = 0; c < c1; ++c) loc1 += gl[c];
  Dev<float> d_parts(2 * rows * d), d_lparts(2 * rows);
  const float scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
  sxa_check(sparse_xattn_fwd(d_q.p, d_k.p, d_v.p, SXA_BF16, static_cast<int32_t>(n_blk), 16,
                             static_cast<int32_t>(hq), static_cast<int32_t>(hkv), static_cast<int32_t>(d),
                             scale, d_anchor.p, d_start.p, d_gs.p, d_gl.p, static_cast<int32_t>(c1), loc1,
                             d_ks.p, d_vs.p, d_parts.p, SXA_F32, d_lparts.p, d_ws.p,
                             static_cast<int64_t>(ws_h.size()), s),
            "sparse_xattn_fwd (first half)");
  sxa_check(sparse_xattn_fwd(d_q.p, d_k.p + loc1 * hkv * d, d_v.p + loc1 * hkv * d, SXA_BF16,
                             static_cast<int32_t>(n_blk), 16, static_cast<int32_t>(hq), static_cast<int32_t>(hkv),
                             static_cast<int32_t>(d), scale, d_anchor.p, d_start.p, d_gs.p + c1, d_gl.p + c1,
                             static_cast<int32_t>(n_chunk - c1), n_loc - loc1, nullptr, nullptr,
                             d_parts.p + rows * d, SXA_F32, d_lparts.p + rows, d_ws.p,
                             static_cast<int64_t>(ws_h.size()), s),
            "sparse_xattn_fwd (second half)");
  Dev<uint16_t> d_o2(rows * d);
  Dev<float> d_lse2(rows);
  sxa_check(lse_combine(d_parts.p, SXA_F32, d_lparts.p, 2, rows, static_cast<int32_t>(d), d_o2.p, SXA_BF16,
                        d_lse2.p, s),
            "lse_combine");
  hip_check(hipStreamSynchronize(s), "sync");
  write_file(dir + "/o2.bin", d_o2.host());
  write_file(dir + "/lse2.bin", d_lse2.host());

  // context_gather: two row ranges of k (rows of hkv * d bf16) back to back
  Dev<int32_t> d_ggs(ggs), d_ggl(ggl);
  const int64_t n_g = static_cast<int64_t>(ggl[0]) + ggl[1];
  Dev<uint16_t> d_kg(n_g * hkv * d);
  sxa_check(context_gather(d_k.p, hkv * d * 2, d_ggs.p, d_ggl.p, 2, n_g, d_kg.p, s), "context_gather");
  hip_check(hipStreamSynchronize(s), "sync");
  write_file(dir + "/kg.bin", d_kg.host());

  // backward of every listed chunk with the own-block term, from the forward's O and lse
  Dev<uint16_t> d_do(dout);
  Dev<float> d_delta(2 * rows), d_dq(rows * d), d_dk(n_loc * hkv * d), d_dv(n_loc * hkv * d);
  Dev<float> d_dks(n_q * hkv * d), d_dvs(n_q * hkv * d);
  Dev<uint8_t> d_bws(static_cast<size_t>(sparse_xattn_bwd_workspace_bytes(
      static_cast<int32_t>(n_blk), n_loc, static_cast<int32_t>(hq), static_cast<int32_t>(hkv), static_cast<int32_t>(d))));
  sxa_check(sparse_xattn_bwd(d_q.p, d_k.p, d_v.p, SXA_BF16, static_cast<int32_t>(n_blk), 16,
                             static_cast<int32_t>(hq), static_cast<int32_t>(hkv), static_cast<int32_t>(d), scale,
                             d_anchor.p, d_start.p, d_gs.p, d_gl.p, static_cast<int32_t>(n_chunk), n_loc, d_ks.p,
                             d_vs.p, d_o.p, d_do.p, d_lse.p, d_delta.p, d_dq.p, d_dk.p, d_dv.p, d_dks.p, d_dvs.p,
                             d_bws.p, static_cast<int64_t>(d_bws.n),
                             SXA_BWD_DELTA | SXA_BWD_DQ | SXA_BWD_DKDV | SXA_BWD_DQ_OVERWRITE, s),
            "sparse_xattn_bwd");
  hip_check(hipStreamSynchronize(s), "sync");
  write_file(dir + "/dq.bin", d_dq.host());
  write_file(dir + "/dk.bin", d_dk.host());
  write_file(dir + "/dv.bin", d_dv.host());
  write_file(dir + "/dks.bin", d_dks.host());
  write_file(dir + "/dvs.bin", d_dvs.host());
  hip_check(hipStreamDestroy(s), "hipStreamDestroy");
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  try {
    return run(argv[1]);
  } catch (const std::exception& e) {
    std::fprintf(stderr, "sxattn_c_driver: %s\n", e.what());
    return 1;
  }
}
