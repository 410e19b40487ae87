// Combine: gate-weighted sum of the expert outputs, plus shared output and residual.
//
// y_s = sum_e G_{s,e} FFN_e(x_s): "MoE技术演进", "GShard" item 3.  The residual
// u_t and the ungated shared experts: "MoE技术演进", "DeepSeekMoE" items 1-2.
// A dropped assignment (row_of < 0) adds nothing; its token keeps the residual
// ("GShard" item 1: overflow passes through the residual connection).
//
// Each thread owns 8 (bf16) or 4 (f32) consecutive columns of one token row and
// accumulates in float32 in a fixed order: residual, shared, then the head's
// assignments j ascending; the sum is rounded once.
#include "common.h"
#include "launch.h"

namespace moe {

template <typename TA>
__global__ __launch_bounds__(256) void combine_kernel(
    const TA *__restrict__ y_perm, const int32_t *__restrict__ row_of, const float *__restrict__ topk_w,
    const TA *__restrict__ res, const TA *__restrict__ sh, TA *__restrict__ y, int T, int H, int k, int dh,
    int tokens_per_block, long r_max) {
  constexpr int EPC = 16 / sizeof(TA);
  const int width = H * dh;
  const int cpr = width / EPC;  // 16-byte chunks per row
  const long t0 = (long)blockIdx.x * tokens_per_block;
  const int nt = (int)min((long)tokens_per_block, (long)T - t0);
  const int K = H * k;
  for (int i = threadIdx.x; i < nt * cpr; i += 256) {
    const int tt = i / cpr, q = i - tt * cpr;
    const long t = t0 + tt;
    const int c0 = q * EPC;
    const int h = c0 / dh;
    float acc[EPC];
#pragma unroll
    for (int v = 0; v < EPC; ++v) acc[v] = 0.f;
    if (res) {
      u32x4 r = reinterpret_cast<const u32x4 *>(res + (size_t)t * width)[q];
      const TA *rv = reinterpret_cast<const TA *>(&r);
#pragma unroll
      for (int v = 0; v < EPC; ++v) acc[v] += Elem<TA>::to_f32(rv[v]);
    }
    if (sh) {
      u32x4 r = reinterpret_cast<const u32x4 *>(sh + (size_t)t * width)[q];
      const TA *rv = reinterpret_cast<const TA *>(&r);
#pragma unroll
      for (int v = 0; v < EPC; ++v) acc[v] += Elem<TA>::to_f32(rv[v]);
    }
    for (int j = h * k; j < (h + 1) * k; ++j) {
      const int row = row_of[t * K + j];
      if (row < 0 || row >= r_max) continue;
      const float w = topk_w[t * K + j];
      u32x4 r = reinterpret_cast<const u32x4 *>(y_perm + (size_t)row * dh + (c0 - h * dh))[0];
      const TA *rv = reinterpret_cast<const TA *>(&r);
#pragma unroll
      for (int v = 0; v < EPC; ++v) acc[v] += w * Elem<TA>::to_f32(rv[v]);
    }
    u32x4 o;
    TA *ov = reinterpret_cast<TA *>(&o);
#pragma unroll
    for (int v = 0; v < EPC; ++v) ov[v] = Elem<TA>::from_f32(acc[v]);
    reinterpret_cast<u32x4 *>(y + (size_t)t * width)[q] = o;
  }
}

int launch_combine(const Shape &s, const void *y_perm, const int32_t *row_of, const float *topk_w,
                   const void *residual, const void *shared_out, void *y, hipStream_t st) {
  const int esz = s.act_f32 ? 4 : 2;
  const long row_bytes = (long)s.H * s.dh * esz;
  long tpb_ = 32768 / row_bytes;
  const int tpb = tpb_ < 1 ? 1 : (int)tpb_;
  const long blocks = ((long)s.T + tpb - 1) / tpb;
  if (blocks == 0) return 0;
  if (s.act_f32)
    hipLaunchKernelGGL(combine_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float *)y_perm, row_of, topk_w,
                       (const float *)residual, (const float *)shared_out, (float *)y, s.T, s.H, s.k, s.dh, tpb, s.R_max);
  else
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st, (const uint16_t *)y_perm, row_of,
                       topk_w, (const uint16_t *)residual, (const uint16_t *)shared_out, (uint16_t *)y, s.T, s.H,
                       s.k, s.dh, tpb, s.R_max);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace moe
