// Standalone use of the Lighthouse C ABI: no PyTorch, only liblighthouse.so
// and the HIP runtime.  Reads a problem from a file, runs lh_forward and
// lh_backward on one stream, and writes the results.
//
// usage: lh_step IN OUT
//   IN : int64 header {B, H, N, d, p, L, S, dtype}, then q, k, v, dout
//        (packed [B,H,N,d], elements of dtype: float32, or bfloat16 bits)
//   OUT: out, dq, dk, dv (dtype, [B,H,N,d]), then int32 sel [B,H,K],
//        sub_idx [B,H,S] and pos [B,H,M]
// Exit status 0 on success; on failure the library's or HIP's message is
// printed and the status is 1.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "lighthouse.h"

namespace {

bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

bool lh_ok(lh_status s, const char* what) {
  if (s == LH_OK) return true;
  std::fprintf(stderr, "%s: status %d: %s\n", what, (int)s, lh_last_error());
  return false;
}

struct Dev {
  void* p = nullptr;
  ~Dev() {
    if (p) (void)hipFree(p);
  }
  bool alloc(size_t n) { return n == 0 || hip_ok(hipMalloc(&p, n), "hipMalloc"); }
};

}  // namespace

int main(int argc, char** argv) {
  // optional third argument "null": run on the default (NULL) stream
  const bool null_stream = argc == 4 && std::string(argv[3]) == "null";
  if (argc != 3 && !null_stream) {
    std::fprintf(stderr, "usage: %s IN OUT [null]\n", argv[0]);
    return 1;
  }
  FILE* fin = std::fopen(argv[1], "rb");
  if (!fin) {
    std::perror(argv[1]);
    return 1;
  }
  int64_t hd[8];
  if (std::fread(hd, sizeof(int64_t), 8, fin) != 8) {
    std::fprintf(stderr, "short header\n");
    return 1;
  }
  lh_shape s = {};  // zero-initialised: packed token tensors
  s.B = hd[0];
  s.H = hd[1];
  s.N = hd[2];
  s.d = hd[3];
  s.p = (int32_t)hd[4];
  s.L = (int32_t)hd[5];
  s.S = hd[6];
  s.dtype = (int32_t)hd[7];
  lh_sizes z;
  if (!lh_ok(lh_query_sizes(&s, &z), "lh_query_sizes")) return 1;
  const size_t tok = z.bytes_qkv;
  std::vector<char> host(4 * tok);
  if (std::fread(host.data(), 1, host.size(), fin) != host.size()) {
    std::fprintf(stderr, "short input\n");
    return 1;
  }
  std::fclose(fin);

  Dev q, k, v, dout, out, dq, dk, dv, ws;
  Dev pq, pk, pv, score, sel, sub_idx, pos, qs, ks, vs, os, lse;
  const size_t wsb = z.ws_forward > z.ws_backward ? z.ws_forward : z.ws_backward;
  bool ok = q.alloc(tok) && k.alloc(tok) && v.alloc(tok) && dout.alloc(tok) && out.alloc(tok) &&
            dq.alloc(tok) && dk.alloc(tok) && dv.alloc(tok) && ws.alloc(wsb) &&
            pq.alloc(z.bytes_pyramid) && pk.alloc(z.bytes_pyramid) && pv.alloc(z.bytes_pyramid) &&
            score.alloc(z.bytes_score) && sel.alloc(z.bytes_sel) && sub_idx.alloc(z.bytes_sub_idx) &&
            pos.alloc(z.bytes_pos) && qs.alloc(z.bytes_sub) && ks.alloc(z.bytes_sub) &&
            vs.alloc(z.bytes_sub) && os.alloc(z.bytes_sub_f32) && lse.alloc(z.bytes_lse);
  if (!ok) return 1;
  Dev* in[4] = {&q, &k, &v, &dout};
  for (int i = 0; i < 4; ++i)
    if (!hip_ok(hipMemcpy(in[i]->p, host.data() + i * tok, tok, hipMemcpyHostToDevice), "copy in"))
      return 1;

  lh_buffers b = {};
  b.pq = pq.p;
  b.pk = pk.p;
  b.pv = pv.p;
  b.score = static_cast<float*>(score.p);
  b.sel = static_cast<int32_t*>(sel.p);
  b.sub_idx = static_cast<int32_t*>(sub_idx.p);
  b.pos = static_cast<int32_t*>(pos.p);
  b.qs = qs.p;
  b.ks = ks.p;
  b.vs = vs.p;
  b.os = static_cast<float*>(os.p);
  b.lse = static_cast<float*>(lse.p);
  hipStream_t st = nullptr;
  if (!null_stream && !hip_ok(hipStreamCreate(&st), "hipStreamCreate")) return 1;
  ok = lh_ok(lh_forward(&s, q.p, k.p, v.p, out.p, &b, ws.p, wsb, st), "lh_forward") &&
       lh_ok(lh_backward(&s, dout.p, &b, dq.p, dk.p, dv.p, ws.p, wsb, st), "lh_backward") &&
       hip_ok(hipStreamSynchronize(st), "hipStreamSynchronize");
  if (st) (void)hipStreamDestroy(st);
  if (!ok) return 1;

  FILE* fo = std::fopen(argv[2], "wb");
  if (!fo) {
    std::perror(argv[2]);
    return 1;
  }
  const Dev* res[4] = {&out, &dq, &dk, &dv};
  for (int i = 0; i < 4; ++i) {
    if (!hip_ok(hipMemcpy(host.data(), res[i]->p, tok, hipMemcpyDeviceToHost), "copy out")) return 1;
    std::fwrite(host.data(), 1, tok, fo);
  }
  const std::pair<const Dev*, size_t> maps[3] = {
      {&sel, z.bytes_sel}, {&sub_idx, z.bytes_sub_idx}, {&pos, z.bytes_pos}};
  for (const auto& m : maps) {
    std::vector<char> h(m.second);
    if (m.second && !hip_ok(hipMemcpy(h.data(), m.first->p, m.second, hipMemcpyDeviceToHost), "copy map"))
      return 1;
    std::fwrite(h.data(), 1, h.size(), fo);
  }
  std::fclose(fo);
  std::printf("lh_step: B=%lld H=%lld N=%lld d=%lld p=%d L=%d S=%lld ok\n", (long long)s.B,
              (long long)s.H, (long long)s.N, (long long)s.d, s.p, s.L, (long long)s.S);
  return 0;
}
