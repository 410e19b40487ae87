// Fused expert MLP for narrow experts (expert input width d_e of 64, 128 or
// 256, bf16): one kernel computes, for a 256-row tile of one expert, the
// gate/up products over d_e, the activation and the down product, with the
// hidden activation never leaving registers.  The expert FFN is the one the
// grouped GEMM path computes: "MoE技术演进", "GShard" item 3 (ReLU experts)
// and "大语言模型并行策略（七）：专家并行", "MoE 模型的参数量分析" (SwiGLU experts).
// Many small experts with few rows each ("挑战三：计算不高效" on the same page) are
// the case it is for.
//
// With d_e this small, the two-launch path (hidden H to HBM, then H W2^T)
// runs tiles whose K is only d_e or d_ff deep: each tile spends more time
// filling and draining its pipeline than on MFMAs, and H makes a round trip
// through HBM.  Here a wave holds its 32 rows of x (all d_e columns) as MFMA
// operands in registers for the whole tile; the block streams each expert's
// weights once per tile, 32 hidden units at a time, through LDS.
//
// Register handoff between the two products: a 16x16x32 MFMA leaves lane
// (r, q) with four consecutive output columns 4q..4q+3 of row r, while the
// next MFMA wants lane (r, q) to hold eight consecutive k (8q..8q+7) of row r.
// Loading the gate/up weight rows of a chunk in the order hidden(f, j) =
// 8 (j / 4) + 4 f + j % 4 (n-fragment f = 0, 1; row j of the fragment) makes
// lane (r, q)'s outputs of fragments 0 and 1 exactly hidden units 8q..8q+7,
// so the activation packs straight into the down product's operand.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int MLP_WAVES = 8, MLP_NT = 64 * MLP_WAVES;
constexpr int MLP_ROWS = 32 * MLP_WAVES;  // rows per block: two 16-row fragments per wave
constexpr int MLP_HC = 32;                // hidden units per chunk

struct MlpArgs {
  const uint16_t *x; long ldx;            // expert input rows (see gather)
  const int32_t *gather; int gK, gEh, gdh; // routed row r = x[gather[r] / gK] + (e / gEh) * gdh, or x[r]
  const uint16_t *w1, *w3, *w2;           // [E][dff][DH], [E][dff][DH] (SwiGLU), [E][DH][dff]
  uint16_t *y; long ldy;                  // y_perm rows [R][DH], or NULL (not written)
  const int32_t *offsets;                 // [E + 1] rows of each expert
  const int32_t *prefix;                  // [E + 1] blocks before each expert
  int E, dff;
  // the folded combine (o != NULL): row r times fw[asg[r]] to o[asg[r] / fK]
  // at column (e / gEh) * DH, row stride ldo
  uint16_t *o; long ldo;
  const float *fw;
  const int32_t *asg;
  int fK;
};

// The folded combine's value of two bf16 outputs packed in a word: the gate
// times each, formed as the combine forms it (0 + w * y in float32, rounded
// once to bf16), so o is bitwise the combine's output.
__device__ __forceinline__ uint32_t mlp_gated(float g, uint32_t v) {
  const float lo = 0.0f + g * bf16_to_f32((uint16_t)(v & 0xFFFFu));
  const float hi = 0.0f + g * bf16_to_f32((uint16_t)(v >> 16));
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}
// Where row r's output goes in o (folded combine): its token's row, its head's slice.
__device__ __forceinline__ uint16_t *mlp_orow(const MlpArgs &p, int e, int a) {
  return p.o + (size_t)(a / p.fK) * p.ldo + (size_t)(e / p.gEh) * p.gdh;
}
// One 16-byte slot (8 bf16, columns 8q ..) of row r's output to y_perm and,
// folded, gated to o.
__device__ __forceinline__ void mlp_put(const MlpArgs &p, int e, int r, int q, u32x4 v) {
  if (p.y) *(u32x4 *)(p.y + (size_t)r * p.ldy + q * 8) = v;
  if (p.o) {
    const int a = p.asg[r];
    const float g = p.fw[a];
    u32x4 u;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = mlp_gated(g, v[c]);
    *(u32x4 *)(mlp_orow(p, e, a) + q * 8) = u;
  }
}

// blocks per expert: ceil(n_e / MLP_ROWS); prefix[e] = blocks before expert e
__global__ __launch_bounds__(1024) void mlp_prefix_kernel(const int32_t *__restrict__ offsets, int E,
                                                          int32_t *__restrict__ prefix) {
  __shared__ int sp[1024];
  const int tid = threadIdx.x, per = (E + 1023) / 1024;
  int nb[8], sum = 0;
  for (int i = 0; i < per && i < 8; ++i) {
    const int e = tid * per + i;
    nb[i] = e < E ? (offsets[e + 1] - offsets[e] + MLP_ROWS - 1) / MLP_ROWS : 0;
    sum += nb[i];
  }
  sp[tid] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int up = tid >= o ? sp[tid - o] : 0;
    __syncthreads();
    sp[tid] += up;
    __syncthreads();
  }
  int run = sp[tid] - sum;
  for (int i = 0; i < per && i < 8; ++i) {
    const int e = tid * per + i;
    if (e < E) prefix[e] = run;
    run += nb[i];
  }
  if (tid == 1023) prefix[E] = sp[1023];
}

// 16-byte slot swizzles.  A ds_read_b128 is served eight lanes at a time
// from a 128-byte bank window (measured: the grouped GEMM's row & 7 swizzle
// of 128-byte rows shows no bank conflict), so the eight lanes that read the
// same logical slot of eight consecutive rows must hit eight distinct 16-byte
// bank groups.  Gate/up rows of RS slots (128 bytes or more) start at the
// same bank: the slot index is XORed with the row's low bits (row & 15 keeps
// row & 7 in the window's slot bits).  Down-weight rows are 64 bytes (4
// slots), two to a window: slot ^ ((row >> 1) & 3).  (With (row >> 2) & 3,
// laid out for a 256-byte window, the multi-head workload's MLP launch
// counted 4.85 M bank-conflict cycles, with this 0.60 M; its time did not
// change.)
template <int RS>
__device__ __forceinline__ int mlp_swz13(int row, int slot) {
  if constexpr (RS >= 16) return slot ^ (row & 15);
  else return slot ^ (row & 7);
}
__device__ __forceinline__ int mlp_swz2(int row, int slot) { return slot ^ ((row >> 1) & 3); }

template <int DH, bool GLU>
struct MlpGeom {
  static constexpr int KST = DH / 32;                  // k-steps of the gate/up products
  static constexpr int RS = DH / 8;                    // 16-byte slots per gate/up weight row
  static constexpr int R13 = GLU ? 2 * MLP_HC : MLP_HC;
  static constexpr int S13 = R13 * RS;                 // slots: the chunk's gate (and up) rows
  static constexpr int S2 = DH * (MLP_HC / 8);         // slots: the chunk's down columns, DH rows of 4
  static constexpr int SST = S13 + S2;                 // slots per stage
  static constexpr int I13 = (S13 + MLP_NT - 1) / MLP_NT, I2 = (S2 + MLP_NT - 1) / MLP_NT;
  static constexpr int NO = DH / 16;                   // output fragments
  static_assert(S13 % 64 == 0 && S2 % 64 == 0, "whole waves per load");
  // every wave issues the same loads per chunk: then a chunk can stay in
  // flight across a barrier (three stages, a counted wait); else two stages
  static constexpr bool UNIFORM = S13 % MLP_NT == 0 && S2 % MLP_NT == 0;
  static constexpr int STAGES = UNIFORM ? 3 : 2;
  static constexpr int LPW = I13 + I2;                 // loads per wave per chunk (UNIFORM)
  static constexpr size_t lds = STAGES * (size_t)SST * 16;
};

template <int DH, bool GLU>
__global__ __launch_bounds__(MLP_NT) void mlp_kernel(MlpArgs p) {
  using G = MlpGeom<DH, GLU>;
  extern __shared__ u32x4 smem[];  // [STAGES][SST]
  const int total = p.prefix[p.E];
  const int b = blockIdx.x;
  if (b >= total) return;
  // blocks go round-robin to the 8 XCDs: a contiguous run of tiles per XCD,
  // so the tiles of one expert share its weights in one L2
  const int q8 = total >> 3;
  const int lt = (b < 8 * q8) ? (b & 7) * q8 + (b >> 3) : b;
  int lo = 0, hi = p.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.prefix[mid] <= lt) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int r0 = p.offsets[e] + (lt - p.prefix[e]) * MLP_ROWS;
  const int M = min(p.offsets[e + 1] - r0, MLP_ROWS);  // rows of this tile (> 0)

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), l16 = lane & 15, cq = lane >> 4;
  const size_t wsz = (size_t)p.dff * DH;
  const uint16_t *W1 = p.w1 + (size_t)e * wsz;
  const uint16_t *W3 = GLU ? p.w3 + (size_t)e * wsz : W1;
  const uint16_t *W2 = p.w2 + (size_t)e * wsz;
  const uint16_t *X = p.x + (p.gather ? (size_t)(e / p.gEh) * p.gdh : 0);

  // this wave's rows of x (clamped into the tile), all DH columns, as MFMA
  // operands: xa[i][ks] = 8 columns 32 ks + 8 cq .. of row 32 w + 16 i + l16
  u32x4 xa[2][G::KST];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = min(32 * w + 16 * i + l16, M - 1), r = r0 + row;
    const size_t src = p.gather ? (size_t)(p.gather[r] / p.gK) : (size_t)r;
    const uint16_t *xr = X + src * p.ldx + 8 * cq;
#pragma unroll
    for (int ks = 0; ks < G::KST; ++ks) xa[i][ks] = *(const u32x4 *)(xr + 32 * ks);
  }

  // The LDS slots this thread fills, as element offsets from the chunk's
  // weights: gate/up rows in the order that hands the activation to the down
  // product in registers (see above), 16-byte slots swizzled as above.  Bit
  // 31 of a gate/up offset: the row is an up row.
  uint32_t o13[G::I13], o2[G::I2];
#pragma unroll
  for (int i = 0; i < G::I13; ++i) {
    const int s = min(i * MLP_NT + tid, G::S13 - 1);
    const int row = s / G::RS, ls = mlp_swz13<G::RS>(row, s % G::RS);
    const int j = row % MLP_HC, f = j / 16, jj = j % 16;
    const int hid = 8 * (jj / 4) + 4 * f + (jj % 4);
    o13[i] = (uint32_t)(hid * DH + 8 * ls) | ((GLU && row >= MLP_HC) ? 0x80000000u : 0u);
  }
#pragma unroll
  for (int i = 0; i < G::I2; ++i) {
    const int s = min(i * MLP_NT + tid, G::S2 - 1);
    const int n = s >> 2, ls = mlp_swz2(n, s & 3);
    o2[i] = (uint32_t)(n * p.dff + 8 * ls);
  }
  // chunk c (hidden units 32 c ..) into stage st
  auto issue = [&](int c, int st) {
    const int h0 = c * MLP_HC;
    const uint16_t *g1 = W1 + (size_t)h0 * DH, *g3 = W3 + (size_t)h0 * DH, *g2 = W2 + h0;
    u32x4 *base = smem + st * G::SST;
#pragma unroll
    for (int i = 0; i < G::I13; ++i)
      if (G::S13 % MLP_NT == 0 || i * MLP_NT + 64 * w < G::S13) {  // wave-uniform
        const uint32_t o = o13[i];
        load_lds16(((o >> 31) ? g3 : g1) + (o & 0x7FFFFFFFu), base + i * MLP_NT + 64 * w);
      }
#pragma unroll
    for (int i = 0; i < G::I2; ++i)
      if (G::S2 % MLP_NT == 0 || i * MLP_NT + 64 * w < G::S2)
        load_lds16(g2 + o2[i], base + G::S13 + i * MLP_NT + 64 * w);
  };

  f32x4 yacc[2][G::NO];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int o = 0; o < G::NO; ++o) yacc[i][o] = f32x4{0.f, 0.f, 0.f, 0.f};

  // NL: m-fragments of this wave that hold rows (wave-uniform); waves past
  // the tile's rows still load and take part in every barrier
  auto run = [&](auto nl) {
    constexpr int NL = decltype(nl)::value;
    const int nch = p.dff / MLP_HC;
    // (a stage past the last chunk gets a copy of it, never read: every wave
    // then has the same loads in flight whatever nch is)
#pragma unroll
    for (int c = 0; c < G::STAGES - 1; ++c) issue(min(c, nch - 1), c);
    // the x rows (loaded before these chunks) are in registers from here on,
    // so no wait inside the loop is for them
    if constexpr (G::UNIFORM) wait_vmcnt<(G::STAGES - 1) * G::LPW>();
    else wait_vmcnt0();
    int st = 0;
    for (int c = 0; c < nch; ++c) {
      // chunk c landed for this wave (the next one may stay in flight), and
      // this wave's LDS reads of the previous chunk are done; the barrier then
      // makes both hold for every wave
      if constexpr (G::UNIFORM) {
        if (c + 1 < nch) wait_vmcnt<G::LPW>(); else wait_vmcnt0();
      } else {
        wait_vmcnt0();
      }
      wait_lgkmcnt0();
      barrier_nofence();
      if (c + G::STAGES - 1 < nch) {
        const int sn = st + G::STAGES - 1;
        issue(c + G::STAGES - 1, sn >= G::STAGES ? sn - G::STAGES : sn);
      }
      if constexpr (NL > 0) {
        const u32x4 *sw = smem + st * G::SST;
        // gate/up in two passes over the chunk's fragments f = 0, 1: pass f
        // leaves lane (l16, cq) with hidden units 8 cq + 4 f .. + 3 of row l16
        u32x4 hf[NL];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          f32x4 ga[NL], ua[NL];
#pragma unroll
          for (int i = 0; i < NL; ++i) {
            ga[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            ua[i] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int ks = 0; ks < G::KST; ++ks) {
            const int phys = mlp_swz13<G::RS>(l16, 4 * ks + cq);  // row 16 f + l16: same swizzle
            const u32x4 wg = sw[(16 * f + l16) * G::RS + phys];
            u32x4 wu;
            if constexpr (GLU) wu = sw[(MLP_HC + 16 * f + l16) * G::RS + phys];
#pragma unroll
            for (int i = 0; i < NL; ++i) {
              ga[i] = mma16(wg, xa[i][ks], ga[i], uint16_t());
              if constexpr (GLU) ua[i] = mma16(wu, xa[i][ks], ua[i], uint16_t());
            }
          }
          // activation, rounded to bf16 like the stored hidden activation
#pragma unroll
          for (int i = 0; i < NL; ++i) {
            float h[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float gt = ga[i][v];
              if constexpr (GLU) h[v] = gt / (1.0f + __expf(-gt)) * ua[i][v];
              else h[v] = fmaxf(gt, 0.0f);
            }
            hf[i][2 * f] = (uint32_t)f32_to_bf16(h[0]) | ((uint32_t)f32_to_bf16(h[1]) << 16);
            hf[i][2 * f + 1] = (uint32_t)f32_to_bf16(h[2]) | ((uint32_t)f32_to_bf16(h[3]) << 16);
          }
        }
        const u32x4 *s2 = sw + G::S13;
#pragma unroll
        for (int o = 0; o < G::NO; ++o) {
          const int n = 16 * o + l16;
          const u32x4 wf = s2[4 * n + mlp_swz2(n, cq)];
#pragma unroll
          for (int i = 0; i < NL; ++i) yacc[i][o] = mma16(wf, hf[i], yacc[i][o], uint16_t());
        }
      }
      st = (st + 1 == G::STAGES) ? 0 : st + 1;
    }
  };
  const int live = M - 32 * w;
  if (live > 16) run(std::integral_constant<int, 2>{});
  else if (live > 0) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 0>{});

  // lane (l16, cq) holds output columns 16 o + 4 cq .. + 3 of row 32 w + 16 i + l16.
  // Where the ring holds a whole output tile, the tile goes out through it:
  // quads into 16-byte slots XOR-swizzled by row (slot q of row r at
  // r * RQY + (q ^ r % RQY)), then whole slots of whole rows per thread; a
  // quad store straight from the registers touches 16 rows for 32 bytes of
  // each per wave instruction.
  constexpr int RQY = DH * 2 / 16;  // 16-byte slots per output row
  if constexpr ((size_t)MLP_ROWS * RQY * 16 <= G::lds && (RQY & (RQY - 1)) == 0) {
    wait_vmcnt0();    // no ring load of this wave still in flight
    wait_lgkmcnt0();  // and its reads of the ring are done
    barrier_nofence();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rt = 32 * w + 16 * i + l16;
#pragma unroll
      for (int o = 0; o < G::NO; ++o) {
        const int ct = 16 * o + 4 * cq;
        uint2 u;
        u.x = (uint32_t)f32_to_bf16(yacc[i][o][0]) | ((uint32_t)f32_to_bf16(yacc[i][o][1]) << 16);
        u.y = (uint32_t)f32_to_bf16(yacc[i][o][2]) | ((uint32_t)f32_to_bf16(yacc[i][o][3]) << 16);
        *(uint2 *)((char *)(smem + rt * RQY + ((ct / 8) ^ (rt % RQY))) + (ct % 8) * 2) = u;
      }
    }
    wait_lgkmcnt0();
    barrier_nofence();
#pragma unroll 4
    for (int s0 = 0; s0 < MLP_ROWS * RQY; s0 += MLP_NT) {
      const int sl = s0 + tid, r = sl / RQY, q = (sl % RQY) ^ (r % RQY);
      if (r < M) mlp_put(p, e, r0 + r, q, smem[sl]);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 32 * w + 16 * i + l16;
    if (row >= M) continue;
    uint16_t *yr = p.y ? p.y + (size_t)(r0 + row) * p.ldy + 4 * cq : nullptr;
    // the folded combine: the row's gate and its slice of o
    float g = 0.f;
    uint16_t *orow = nullptr;
    if (p.o) {
      const int a = p.asg[r0 + row];
      g = p.fw[a];
      orow = mlp_orow(p, e, a) + 4 * cq;
    }
#pragma unroll
    for (int o = 0; o < G::NO; ++o) {
      uint2 u;
      u.x = (uint32_t)f32_to_bf16(yacc[i][o][0]) | ((uint32_t)f32_to_bf16(yacc[i][o][1]) << 16);
      u.y = (uint32_t)f32_to_bf16(yacc[i][o][2]) | ((uint32_t)f32_to_bf16(yacc[i][o][3]) << 16);
      if (yr) *(uint2 *)(yr + 16 * o) = u;
      if (orow) *(uint2 *)(orow + 16 * o) = make_uint2(mlp_gated(g, u.x), mlp_gated(g, u.y));
    }
  }
}

bool mlp_fused_supported(const Shape &s) {
  return !s.act_f32 && (s.dh == 64 || s.dh == 128 || s.dh == 256) && s.dff > 0 && s.dff % MLP_HC == 0 &&
         s.E <= 8192;
}

// Layers whose combine the fused MLP can do: multi-head latent layers (the
// combine writes o with no residual or shared part) where every (token, head)
// keeps its one choice (top-1 per head, nothing dropped), so each slice of o
// is one gated expert row.
bool fold_supported(const Shape &s) {
  return mlp_fused_supported(s) && s.latent && s.k == 1 && s.drop == DROP_NONE && !s.expert_choice &&
         s.n_shared == 0;
}

template <int DH, bool GLU>
static int run_mlp(const MlpArgs &a, long grid, hipStream_t st) {
  constexpr size_t lds = MlpGeom<DH, GLU>::lds;
  static_assert(lds <= 160 * 1024, "LDS per workgroup");
  hipLaunchKernelGGL((mlp_kernel<DH, GLU>), dim3((unsigned)grid), dim3(MLP_NT), lds, st, a);
  return launch_status("fused expert mlp");
}

int launch_mlp_fused(const Shape &s, const void *xin, const int32_t *gather, const int32_t *offsets, const void *w1,
                     const void *w3, const void *w2, void *y_perm, int32_t *prefix, hipStream_t st,
                     const FoldOut &fold) {
  if (!mlp_fused_supported(s)) return -2;
  if (fold.o && !fold_supported(s)) return -2;
  if (!fold.o && !y_perm && s.R_max) return -1;
  hipLaunchKernelGGL(mlp_prefix_kernel, dim3(1), dim3(1024), 0, st, offsets, s.E, prefix);
  if (int rc = launch_status("fused mlp prefix")) return rc;
  MlpArgs a{};
  a.x = (const uint16_t *)xin; a.ldx = gather ? (long)s.H * s.dh : s.dh;
  a.gather = gather; a.gK = s.K; a.gEh = s.Eh; a.gdh = s.dh;
  a.w1 = (const uint16_t *)w1; a.w3 = (const uint16_t *)w3; a.w2 = (const uint16_t *)w2;
  a.y = (uint16_t *)y_perm; a.ldy = s.dh;
  a.offsets = offsets; a.prefix = prefix; a.E = s.E; a.dff = s.dff;
  a.o = (uint16_t *)fold.o; a.ldo = (long)s.H * s.dh; a.fw = fold.w; a.asg = fold.asg; a.fK = s.K;
  const long grid = (s.R_max + MLP_ROWS - 1) / MLP_ROWS + s.E;  // blocks past the prefix total exit
  const bool glu = s.act == 1;
  switch (s.dh) {
    case 64: return glu ? run_mlp<64, true>(a, grid, st) : run_mlp<64, false>(a, grid, st);
    case 128: return glu ? run_mlp<128, true>(a, grid, st) : run_mlp<128, false>(a, grid, st);
    default: return glu ? run_mlp<256, true>(a, grid, st) : run_mlp<256, false>(a, grid, st);
  }
}

}  // namespace moe
