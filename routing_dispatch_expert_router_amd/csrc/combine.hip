// Combine: gate-weighted sum of the expert outputs, plus shared output and residual.
//
// y_s = sum_e G_{s,e} FFN_e(x_s): "MoE技术演进", "GShard" item 3.  The residual
// u_t and the ungated shared experts: "MoE技术演进", "DeepSeekMoE" items 1-2.
// A dropped assignment (row_of < 0) adds nothing; its token keeps the residual
// ("GShard" item 1: overflow passes through the residual connection).
//
// Each thread owns 8 (bf16) or 4 (f32) consecutive columns of one token row and
// accumulates in float32 in a fixed order: residual, shared, then the head's
// assignments j ascending; the sum is rounded once.  The expert rows and the
// residual are read once and the output written once, so those accesses are
// non-temporal (streamed past the caches): measured on MI355X, the
// group-limited layer's combine 135 -> 126 us from cold caches (139 -> 110
// back to back) and the coarse layer's 28.2 -> 26.7 us cold (21.7 -> 23.3 us
// back to back).
#include "common.h"
#include "launch.h"

namespace moe {

// One thread per 16 bytes of an output row (grid-stride over T x chunks).  KH
// (>= the choices per head) is a compile-time bound so every expert-row load
// of the token is issued before the first add.  WU: a head's row holds a multiple of 64
// chunks, so the 64 lanes of a wave share one token and head (grid strides are
// multiples of 64) and its row indices and gates are read once per wave, as
// scalar loads.
template <typename TA, int KH, bool WU>
__global__ __launch_bounds__(256) void combine_kernel(
    const TA *__restrict__ y_perm, const int32_t *__restrict__ row_of, const float *__restrict__ topk_w,
    const TA *__restrict__ res, const TA *__restrict__ sh, TA *__restrict__ y, int T, int H, int k, int dh,
    long r_max) {
  constexpr int EPC = 16 / sizeof(TA);
  const int width = H * dh;
  const int cpr = width / EPC;  // 16-byte chunks per row
  const int K = H * k;
  const long total = (long)T * cpr;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    long t = i / cpr;
    const int q = (int)(i - t * cpr);
    const int c0 = q * EPC;
    int h = c0 / dh;
    if constexpr (WU) {
      t = __builtin_amdgcn_readfirstlane((int)t);
      h = __builtin_amdgcn_readfirstlane(h);
    }
    constexpr int KA = KH > 0 ? KH : 1;  // KH == 0: a runtime loop over k (expert choice)
    int row[KA];
    float w[KA];
    u32x4 v[KA];
    if constexpr (KH > 0) {
#pragma unroll
      for (int j = 0; j < KH; ++j) {
        row[j] = -1;
        w[j] = 0.f;
        if (j < k) {
          const int r = row_of[t * K + h * k + j];
          row[j] = (r >= 0 && r < r_max) ? r : -1;
          w[j] = topk_w[t * K + h * k + j];
        }
      }
      // a dropped slot loads nothing (a stand-in address would cost HBM reads
      // when many slots are dropped)
#pragma unroll
      for (int j = 0; j < KH; ++j)
        v[j] = row[j] >= 0 ? __builtin_nontemporal_load(
                                 reinterpret_cast<const u32x4 *>(y_perm + (size_t)row[j] * dh + (c0 - h * dh)))
                           : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 rv = res ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(res + (size_t)t * width) + q)
                   : u32x4{0u, 0u, 0u, 0u};
    u32x4 sv = sh ? reinterpret_cast<const u32x4 *>(sh + (size_t)t * width)[q] : u32x4{0u, 0u, 0u, 0u};
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    // fixed order: residual, shared, then the head's choices j ascending
    if (res) {
      const TA *p = reinterpret_cast<const TA *>(&rv);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += Elem<TA>::to_f32(p[e]);
    }
    if (sh) {
      const TA *p = reinterpret_cast<const TA *>(&sv);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += Elem<TA>::to_f32(p[e]);
    }
    if constexpr (KH > 0) {
#pragma unroll
      for (int j = 0; j < KH; ++j) {
        const TA *p = reinterpret_cast<const TA *>(&v[j]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const float a = acc[e] + w[j] * Elem<TA>::to_f32(p[e]);
          acc[e] = row[j] >= 0 ? a : acc[e];  // a dropped slot adds nothing
        }
      }
    } else {
      // slots scanned four at a time (16-byte loads) when the row allows it
      const int32_t *ro = row_of + t * K + h * k;
      const bool vec = (k & 3) == 0 && ((uintptr_t)ro & 15) == 0;
      for (int j0 = 0; j0 < k; j0 += 4) {
        int r4[4];
        if (vec) {
          const int4 q4 = *reinterpret_cast<const int4 *>(ro + j0);
          r4[0] = q4.x; r4[1] = q4.y; r4[2] = q4.z; r4[3] = q4.w;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) r4[u] = j0 + u < k ? ro[j0 + u] : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = r4[u];
          if (r < 0 || r >= r_max) continue;
          const float wj = topk_w[t * K + h * k + j0 + u];
          const u32x4 vj = reinterpret_cast<const u32x4 *>(y_perm + (size_t)r * dh + (c0 - h * dh))[0];
          const TA *p = reinterpret_cast<const TA *>(&vj);
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[e] += wj * Elem<TA>::to_f32(p[e]);
        }
      }
    }
    u32x4 o;
    TA *ov = reinterpret_cast<TA *>(&o);
#pragma unroll
    for (int e = 0; e < EPC; ++e) ov[e] = Elem<TA>::from_f32(acc[e]);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(y + (size_t)t * width) + q);
  }
}

template <typename TA, int KH>
static void launch_c(const Shape &s, const void *y_perm, const int32_t *row_of, const float *topk_w,
                     const void *residual, const void *shared_out, void *y, hipStream_t st) {
  const long total = (long)s.T * (s.H * s.dh * (long)sizeof(TA) / 16);
  long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const bool wu = (s.dh * (long)sizeof(TA) / 16) % 64 == 0;  // a head's chunks fill whole waves
  if (wu)
    hipLaunchKernelGGL((combine_kernel<TA, KH, true>), dim3(blocks), dim3(256), 0, st, (const TA *)y_perm, row_of,
                       topk_w, (const TA *)residual, (const TA *)shared_out, (TA *)y, s.T, s.H, s.k, s.dh, s.R_max);
  else
    hipLaunchKernelGGL((combine_kernel<TA, KH, false>), dim3(blocks), dim3(256), 0, st, (const TA *)y_perm, row_of,
                       topk_w, (const TA *)residual, (const TA *)shared_out, (TA *)y, s.T, s.H, s.k, s.dh, s.R_max);
}

template <typename TA>
static void launch_typed(const Shape &s, const void *y_perm, const int32_t *row_of, const float *topk_w,
                         const void *residual, const void *shared_out, void *y, hipStream_t st) {
  if (s.k <= 1) launch_c<TA, 1>(s, y_perm, row_of, topk_w, residual, shared_out, y, st);
  else if (s.k <= 2) launch_c<TA, 2>(s, y_perm, row_of, topk_w, residual, shared_out, y, st);
  else if (s.k <= 4) launch_c<TA, 4>(s, y_perm, row_of, topk_w, residual, shared_out, y, st);
  else if (s.k <= 8) launch_c<TA, 8>(s, y_perm, row_of, topk_w, residual, shared_out, y, st);
  else launch_c<TA, 0>(s, y_perm, row_of, topk_w, residual, shared_out, y, st);
}

int launch_combine(const Shape &s, const void *y_perm, const int32_t *row_of, const float *topk_w,
                   const void *residual, const void *shared_out, void *y, hipStream_t st) {
  if (s.T == 0) return 0;
  if (s.act_f32)
    launch_typed<float>(s, y_perm, row_of, topk_w, residual, shared_out, y, st);
  else
    launch_typed<uint16_t>(s, y_perm, row_of, topk_w, residual, shared_out, y, st);
  return launch_status("combine");
}

}  // namespace moe
