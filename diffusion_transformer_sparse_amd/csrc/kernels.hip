// gfx950 kernels of the hierarchical local attention path and their C-ABI
// launchers: window-first permutation (and its inverse), in-place 2D axial
// RoPE, and the composite-masked block-sparse attention forward.
//
// Method: "UltraGen: Efficient Ultra-High-Resolution Image Generation with
// Hierarchical Local Attention" (papernotes.org notes, 关键设计 1-3; the
// gist.science summary, section 2.A-2.B).  The kernel design is our own for
// CDNA4; the FlashAttention-2 / SageAttention tile sizes the pages mention
// are not used.
//
// Tensor layout everywhere: [B, L, Hh, D] contiguous, D innermost, so one
// token's row of all heads is Hh*D contiguous elements.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>
#include <type_traits>

#include "plan_internal.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Row gather: dst row j <- src row map(j), whole token rows (all heads) at a
// time, 16-byte vectors.  Rows outside [T, T+N) (text, LR) copy in place;
// HR row T+i copies from T + table[i].  With table = perm this is the
// window-first permutation, with table = inverse it is the unpermutation.
// Pure HBM streaming: every byte is read once and written once.
// ---------------------------------------------------------------------------
constexpr int kGatherThreads = 256;
constexpr int kGatherRows = 8;     // token rows per workgroup
constexpr int kGatherUnroll = 4;   // 16-B loads in flight per thread

__global__ __launch_bounds__(kGatherThreads) void row_gather_kernel(const uint4* __restrict__ src,
                                                                     uint4* __restrict__ dst, int32_t L, int32_t T,
                                                                     int32_t N, int32_t units,
                                                                     const int32_t* __restrict__ table) {
  const int64_t batch_units = int64_t(L) * units;
  src += blockIdx.y * batch_units;
  dst += blockIdx.y * batch_units;
  const int32_t row0 = blockIdx.x * kGatherRows;
  const int32_t nrows = min(kGatherRows, L - row0);
  const int32_t total = nrows * units;
  for (int32_t base = threadIdx.x; base < total; base += kGatherThreads * kGatherUnroll) {
    uint4 v[kGatherUnroll];
    int64_t doff[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int32_t f = base + u * kGatherThreads;
      doff[u] = -1;
      if (f < total) {
        const int32_t r = f / units;
        const int32_t c = f - r * units;
        const int32_t j = row0 + r;
        const int32_t s = (j >= T && j < T + N) ? T + table[j - T] : j;
        v[u] = src[int64_t(s) * units + c];
        doff[u] = int64_t(j) * units + c;
      }
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u)
      if (doff[u] >= 0) dst[doff[u]] = v[u];
  }
}

// ---------------------------------------------------------------------------
// 2D axial RoPE, in place on permuted Q and K (关键设计 1-2).  Row j of the
// permuted sequence: HR slot j-T holds raster token perm[j-T] = (r, c); LR row
// T+N+i holds LR token (m, n) = (i / w, i % w) at position (rho*m, rho*n).
// Dims [0, D/2) turn by the row position, [D/2, D) by the column position;
// pair (2k, 2k+1) of a half turns by pos * omega_k, (cos, sin) from the
// plan's table cs[pos][k].  Each thread owns one 16-byte vector of one head
// row in both Q and K.
// ---------------------------------------------------------------------------
constexpr int kRopeThreads = 256;

template <typename T>
__global__ __launch_bounds__(kRopeThreads) void rope2d_kernel(T* __restrict__ q, T* __restrict__ k, int32_t L,
                                                              int32_t T0, int32_t N, int32_t W, int32_t lr_w,
                                                              int32_t rho, int32_t heads, int32_t D,
                                                              const int32_t* __restrict__ perm,
                                                              const float2* __restrict__ cs) {
  constexpr int E = 16 / sizeof(T);  // elements per thread (8 bf16 or 4 fp32)
  const int32_t units_per_head = D / E;
  const int32_t units = heads * units_per_head;
  const int64_t rows = int64_t(L - T0);  // HR + LR rows
  const int64_t f = int64_t(blockIdx.x) * kRopeThreads + threadIdx.x;
  if (f >= rows * units) return;
  const int32_t rr = int32_t(f / units);
  const int32_t c = int32_t(f - int64_t(rr) * units);
  const int32_t j = T0 + rr;
  int32_t pr, pc;
  if (rr < N) {
    const int32_t idx = perm[rr];
    pr = idx / W;
    pc = idx - pr * W;
  } else {
    const int32_t i = rr - N;
    const int32_t m = i / lr_w;
    pr = rho * m;
    pc = rho * (i - m * lr_w);
  }
  const int32_t e0 = (c % units_per_head) * E;  // first dim of this vector
  const int32_t half = D / 2;
  const int32_t pos = e0 < half ? pr : pc;
  const int32_t k0 = (e0 < half ? e0 : e0 - half) / 2;  // first pair index
  const float2* tab = cs + int64_t(pos) * (D / 4) + k0;
  const int64_t off = (int64_t(blockIdx.y) * L + j) * units + c;  // in 16-B units
  uint4* qv = reinterpret_cast<uint4*>(q) + off;
  uint4* kv = reinterpret_cast<uint4*>(k) + off;
  uint4 qa = *qv, ka = *kv;
  if constexpr (std::is_same<T, float>::value) {
    const float2 t0 = tab[0], t1 = tab[1];
    float* x = reinterpret_cast<float*>(&qa);
    float* y = reinterpret_cast<float*>(&ka);
    const float2 t[2] = {t0, t1};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float a = x[2 * p], b = x[2 * p + 1];
      x[2 * p] = a * t[p].x - b * t[p].y;
      x[2 * p + 1] = a * t[p].y + b * t[p].x;
      const float a2 = y[2 * p], b2 = y[2 * p + 1];
      y[2 * p] = a2 * t[p].x - b2 * t[p].y;
      y[2 * p + 1] = a2 * t[p].y + b2 * t[p].x;
    }
  } else {
    float2 t[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) t[p] = tab[p];
    bf16x8 x = *reinterpret_cast<bf16x8*>(&qa);
    bf16x8 y = *reinterpret_cast<bf16x8*>(&ka);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float a = float(x[2 * p]), b = float(x[2 * p + 1]);
      x[2 * p] = __bf16(a * t[p].x - b * t[p].y);
      x[2 * p + 1] = __bf16(a * t[p].y + b * t[p].x);
      const float a2 = float(y[2 * p]), b2 = float(y[2 * p + 1]);
      y[2 * p] = __bf16(a2 * t[p].x - b2 * t[p].y);
      y[2 * p + 1] = __bf16(a2 * t[p].y + b2 * t[p].x);
    }
    qa = *reinterpret_cast<uint4*>(&x);
    ka = *reinterpret_cast<uint4*>(&y);
  }
  *qv = qa;
  *kv = ka;
}

// ---------------------------------------------------------------------------
// Composite-masked attention forward (关键设计 3 with the mask of 关键设计 2).
//
// One workgroup = one query tile (<= 256 permuted rows sharing one key set)
// of one (batch, head); 8 waves x 32 queries.  The key set is a list of
// contiguous row ranges, walked in 64-key tiles staged through LDS (double
// buffered, one barrier per tile).
//
// Per wave and 64-key tile, with 32x32 MFMA tiles (lane l: column l%32,
// lane half g = l/32):
//   S^T = K Q^T    A = K rows from LDS, B = the wave's Q held in registers.
//                  Output lane l holds query l%32 and 16 keys
//                  8*(j/4) + 4*g + j%4 (j < 16) of each 32-key block, so a
//                  query's softmax statistics are lane-local except for one
//                  exchange between the two lane halves.
//   P = exp2(S*scale*log2e - m), m the running maximum (fp32).
//   O^T += V^T P^T A = V^T from LDS, B = P^T straight from the S^T
//                  registers.  V is stored transposed in LDS with its 4-key
//                  groups reordered so that each lane's 8 B-operand keys are
//                  the 8 keys its S^T registers hold: no register shuffles.
// The running maximum is only moved when a tile's maximum exceeds it by more
// than 8 (log2 units); the final normalisation uses the same reference, so
// the result is unchanged while the 64 O^T registers are rescaled rarely.
// bf16: v_mfma_f32_32x32x16_bf16, P rounded to bf16 for the PV product and
// the row sum taken over the same rounded P; fp32: v_mfma_f32_32x32x2_f32.
// ---------------------------------------------------------------------------
constexpr int kAttnThreads = 512;
constexpr int kKT = ug::kAttnKeyTile;  // 64

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t row_stride;    // elements between consecutive rows (Hh*D)
  int64_t batch_stride;  // elements between consecutive batches (L*Hh*D)
  int32_t heads;
  int32_t pad;
  const ug::Task* tasks;
  const ug::Range* ranges;
  const ug::Block* blocks;
  float scale_log2;      // log2(e) / sqrt(D)
};

template <typename T, int D>
struct AttnLds {
  static constexpr bool kBF = std::is_same<T, __bf16>::value;
  // K rows [key][dim], padded by 16 bytes so 32 lanes reading 32 rows hit
  // distinct banks.
  static constexpr int kKStride = D + 16 / int(sizeof(T));
  // bf16: V^T rows [dim][key position]; fp32: V rows [key][dim].
  static constexpr int kVStride = kBF ? (kKT + 8) : (D + 4);
  static constexpr int kKElems = kKT * kKStride;
  static constexpr int kVElems = kBF ? D * kVStride : kKT * kVStride;
  static constexpr int kStageElems = kKElems + kVElems;
  static constexpr int kBytes = 2 * kStageElems * int(sizeof(T));
  // staging work per thread
  static constexpr int kKChunks = kKT * D * int(sizeof(T)) / 16;      // 16-B chunks of K
  static constexpr int kKPerThread = (kKChunks + kAttnThreads - 1) / kAttnThreads;
  static constexpr int kVUnits = kBF ? (kKT / 4) * (D / 4) : kKChunks;  // bf16: 4 keys x 4 dims
  static constexpr int kVPerThread = (kVUnits + kAttnThreads - 1) / kAttnThreads;
};

__device__ __forceinline__ float wave_other_half(float x) { return __shfl_xor(x, 32); }

template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_fwd_kernel(AttnParams p) {
  using Lds = AttnLds<T, D>;
  constexpr bool kBF = Lds::kBF;
  __shared__ __attribute__((aligned(16))) T smem[2 * Lds::kStageElems];

  const ug::Block blk = p.blocks[blockIdx.x];
  if (blk.task < 0) return;  // idle workgroup (uniform)
  const ug::Task task = p.tasks[blk.task];
  const int32_t b = blk.bh / p.heads, h = blk.bh - b * p.heads;
  const int64_t hoff = int64_t(b) * p.batch_stride + int64_t(h) * D;
  const T* __restrict__ qg = static_cast<const T*>(p.q) + hoff;
  const T* __restrict__ kg = static_cast<const T*>(p.k) + hoff;
  const T* __restrict__ vg = static_cast<const T*>(p.v) + hoff;
  T* __restrict__ og = static_cast<T*>(p.o) + hoff;
  const int64_t rs = p.row_stride;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int32_t qrow = task.q0 + wave * 32 + l32;
  const bool qvalid = qrow < task.q1;
  const bool wave_active = task.q0 + wave * 32 < task.q1;  // uniform per wave
  const int32_t qload = qvalid ? qrow : task.q1 - 1;

  // The wave's queries as the B operand of S^T = K Q^T.
  constexpr int kQRegs = kBF ? D / 16 : D / 2;
  using QReg = typename std::conditional<kBF, bf16x8, float>::type;
  QReg qf[kQRegs];
#pragma unroll
  for (int i = 0; i < kQRegs; ++i) {
    if constexpr (kBF)
      qf[i] = *reinterpret_cast<const bf16x8*>(qg + qload * rs + 16 * i + 8 * g);
    else
      qf[i] = qg[qload * rs + 2 * i + g];
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[t][j] = 0.f;
  float m2 = -INFINITY;  // running maximum, in log2 units (scaled)
  float lsum = 0.f;      // this lane half's share of the row sum

  // ---- staging: global -> registers -> LDS
  uint4 kreg[Lds::kKPerThread];
  typename std::conditional<kBF, uint2, uint4>::type vreg[kBF ? 4 * Lds::kVPerThread : Lds::kVPerThread];

  auto load_tile = [&](int32_t ks, int32_t nv) {
#pragma unroll
    for (int i = 0; i < Lds::kKPerThread; ++i) {
      const int c = tid + i * kAttnThreads;
      if (c < Lds::kKChunks) {
        constexpr int cpr = D * int(sizeof(T)) / 16;  // chunks per row
        const int r = c / cpr, cc = c - (c / cpr) * cpr;
        const int32_t row = ks + min(r, nv - 1);
        kreg[i] = *reinterpret_cast<const uint4*>(kg + row * rs + cc * (16 / int(sizeof(T))));
      }
    }
    if constexpr (kBF) {
#pragma unroll
      for (int i = 0; i < Lds::kVPerThread; ++i) {
        const int u = tid + i * kAttnThreads;
        if (u < Lds::kVUnits) {
          const int kgp = u & 15, dq = u >> 4;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int32_t row = ks + min(4 * kgp + r, nv - 1);
            vreg[4 * i + r] = *reinterpret_cast<const uint2*>(vg + row * rs + 4 * dq);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < Lds::kVPerThread; ++i) {
        const int c = tid + i * kAttnThreads;
        if (c < Lds::kVUnits) {
          constexpr int cpr = D * int(sizeof(T)) / 16;
          const int r = c / cpr, cc = c - (c / cpr) * cpr;
          const int32_t row = ks + min(r, nv - 1);
          vreg[i] = *reinterpret_cast<const uint4*>(vg + row * rs + cc * 4);
        }
      }
    }
  };

  auto store_tile = [&](T* stage) {
    T* ks_ = stage;
    T* vs_ = stage + Lds::kKElems;
#pragma unroll
    for (int i = 0; i < Lds::kKPerThread; ++i) {
      const int c = tid + i * kAttnThreads;
      if (c < Lds::kKChunks) {
        constexpr int cpr = D * int(sizeof(T)) / 16;
        const int r = c / cpr, cc = c - (c / cpr) * cpr;
        *reinterpret_cast<uint4*>(ks_ + r * Lds::kKStride + cc * (16 / int(sizeof(T)))) = kreg[i];
      }
    }
    if constexpr (kBF) {
#pragma unroll
      for (int i = 0; i < Lds::kVPerThread; ++i) {
        const int u = tid + i * kAttnThreads;
        if (u < Lds::kVUnits) {
          const int kgp = u & 15, dq = u >> 4;
          // key group kgp of 4 keys -> position group: chunk kgp/4 of 16
          // positions, in-chunk group order (0, 2, 1, 3) so that lane half g
          // finds keys {4g..4g+3, 8+4g..8+4g+3} at positions 8g..8g+7.
          const int sub = kgp & 3;
          const int pg = (sub == 1) ? 2 : (sub == 2) ? 1 : sub;
          const int pos = (kgp >> 2) * 16 + pg * 4;
          const uint2 r0 = vreg[4 * i + 0], r1 = vreg[4 * i + 1], r2 = vreg[4 * i + 2], r3 = vreg[4 * i + 3];
          // 4x4 transpose of 16-bit values: dim e gets keys 0..3 of the group.
          auto lo2 = [](uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); };
          auto hi2 = [](uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); };
          const uint2 o0 = make_uint2(lo2(r0.x, r1.x), lo2(r2.x, r3.x));
          const uint2 o1 = make_uint2(hi2(r0.x, r1.x), hi2(r2.x, r3.x));
          const uint2 o2 = make_uint2(lo2(r0.y, r1.y), lo2(r2.y, r3.y));
          const uint2 o3 = make_uint2(hi2(r0.y, r1.y), hi2(r2.y, r3.y));
          T* base = vs_ + (4 * dq) * Lds::kVStride + pos;
          *reinterpret_cast<uint2*>(base + 0 * Lds::kVStride) = o0;
          *reinterpret_cast<uint2*>(base + 1 * Lds::kVStride) = o1;
          *reinterpret_cast<uint2*>(base + 2 * Lds::kVStride) = o2;
          *reinterpret_cast<uint2*>(base + 3 * Lds::kVStride) = o3;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < Lds::kVPerThread; ++i) {
        const int c = tid + i * kAttnThreads;
        if (c < Lds::kVUnits) {
          constexpr int cpr = D * int(sizeof(T)) / 16;
          const int r = c / cpr, cc = c - (c / cpr) * cpr;
          *reinterpret_cast<uint4*>(vs_ + r * Lds::kVStride + cc * 4) = vreg[i];
        }
      }
    }
  };

  auto compute = [&](const T* stage, int32_t nv) {
    const T* ks_ = stage;
    const T* vs_ = stage + Lds::kKElems;
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[mb][j] = 0.f;
      const T* krow = ks_ + (mb * 32 + l32) * Lds::kKStride;
#pragma unroll
      for (int i = 0; i < kQRegs; ++i) {
        if constexpr (kBF) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * i + 8 * g);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i], s[mb], 0, 0, 0);
        } else {
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * i + g], qf[i], s[mb], 0, 0, 0);
        }
      }
    }
    if (nv < kKT) {  // ragged tail of a key range (uniform)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (mb * 32 + 8 * (j >> 2) + 4 * g + (j & 3) >= nv) s[mb][j] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[mb][j]);
    mx = fmaxf(mx, wave_other_half(mx));
    const float mt = mx * p.scale_log2;
    const bool need = mt > m2 + 8.0f;
    if (__ballot(need)) {
      const float mnew = need ? mt : m2;
      const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
      m2 = mnew;
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[t][j] *= alpha;
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[mb][j] = __builtin_amdgcn_exp2f(fmaf(s[mb][j], p.scale_log2, -m2));

    if constexpr (kBF) {
      bf16x8 pb[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[c][e] = __bf16(s[c >> 1][(c & 1) * 8 + e]);
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 ones = {__bf16(1.0f), __bf16(1.0f)};
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pb[c][e], pb[c][e + 1]};
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
        }
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        const T* vrow = vs_ + (t * 32 + l32) * Lds::kVStride;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + 16 * c + 8 * g);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], acc[t], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) lsum += s[mb][j];
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = mb * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs_[key * Lds::kVStride + t * 32 + l32], s[mb][j],
                                                          acc[t], 0, 0, 0);
          }
    }
  };

  // ---- walk the key ranges in 64-key tiles
  int32_t ri = task.r0;
  ug::Range cur = p.ranges[ri];
  int32_t ks = cur.k0;
  auto advance = [&]() {
    ks += kKT;
    if (ks >= cur.k1) {
      ++ri;
      if (ri < task.r1) {
        cur = p.ranges[ri];
        ks = cur.k0;
      }
    }
  };

  int32_t nv = min(kKT, cur.k1 - ks);
  load_tile(ks, nv);
  store_tile(smem);
  __syncthreads();
  advance();
  for (int it = 0;; ++it) {
    const bool has_next = ri < task.r1;
    int32_t nv_next = 0;
    if (has_next) {
      nv_next = min(kKT, cur.k1 - ks);
      load_tile(ks, nv_next);
    }
    if (wave_active) compute(smem + (it & 1) * Lds::kStageElems, nv);
    if (!has_next) break;
    store_tile(smem + ((it + 1) & 1) * Lds::kStageElems);
    __syncthreads();
    nv = nv_next;
    advance();
  }

  // ---- epilogue: combine the two lane halves' row sums, normalise, store
  const float ltot = lsum + wave_other_half(lsum);
  if (!wave_active || !qvalid) return;
  const float inv = 1.0f / ltot;
  T* orow = og + qrow * rs;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = t * 32 + 8 * q4 + 4 * g;
      if constexpr (kBF) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = __bf16(acc[t][4 * q4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + d0) = w;
      } else {
        float4 w = make_float4(acc[t][4 * q4 + 0] * inv, acc[t][4 * q4 + 1] * inv, acc[t][4 * q4 + 2] * inv,
                               acc[t][4 * q4 + 3] * inv);
        *reinterpret_cast<float4*>(orow + d0) = w;
      }
    }
}

// ---------------------------------------------------------------------------
// launcher helpers
// ---------------------------------------------------------------------------
ug_status check_plan(ug_plan_t p, const char* fn) {
  if (!p) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": plan is NULL");
  if (p->host_only) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": plan was built host-only");
  return UG_OK;
}

bool aligned16(const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; }

int64_t tensor_bytes(ug_plan_t p) {
  return int64_t(p->d.batch) * p->L * p->d.heads * p->d.head_dim * (p->d.dtype == UG_BF16 ? 2 : 4);
}

bool overlap(const void* a, const void* b, int64_t n) {
  const auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + uintptr_t(n) && y < x + uintptr_t(n);
}

ug_status launch_status(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return ug::fail(UG_ERR_HIP, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
  return UG_OK;
}

int current_device() {
  int d = -1;
  if (hipGetDevice(&d) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return d;
}

ug_status gather(ug_plan_t p, const void* src, void* dst, const int32_t* table, hipStream_t s, const char* fn) {
  ug::clear_error();
  ug_status st = check_plan(p, fn);
  if (st != UG_OK) return st;
  if (!src || !dst) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": NULL tensor");
  if (!aligned16(src) || !aligned16(dst))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": tensors must be 16-byte aligned");
  if (overlap(src, dst, tensor_bytes(p)))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": input and output overlap (out of place only)");
  if (current_device() != p->device)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": current device is not the plan's device");
  const int32_t units = int32_t(int64_t(p->d.heads) * p->d.head_dim * (p->d.dtype == UG_BF16 ? 2 : 4) / 16);
  const dim3 grid(unsigned((p->L + kGatherRows - 1) / kGatherRows), unsigned(p->d.batch));
  hipLaunchKernelGGL(row_gather_kernel, grid, dim3(kGatherThreads), 0, s, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), int32_t(p->L), int32_t(p->T), int32_t(p->N), units, table);
  return launch_status(fn);
}

template <typename T, int D>
void launch_attn(ug_plan_t p, const AttnParams& ap, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<T, D>), dim3(unsigned(p->blocks.size())), dim3(kAttnThreads), 0, s, ap);
}

}  // namespace

extern "C" {

ug_status ug_permute(ug_plan_t p, const void* x_raster, void* x_perm, void* stream) {
  return gather(p, x_raster, x_perm, p ? p->d_perm : nullptr, static_cast<hipStream_t>(stream), "ug_permute");
}

ug_status ug_unpermute(ug_plan_t p, const void* x_perm, void* x_raster, void* stream) {
  return gather(p, x_perm, x_raster, p ? p->d_inv : nullptr, static_cast<hipStream_t>(stream), "ug_unpermute");
}

ug_status ug_rope2d(ug_plan_t p, void* q_perm, void* k_perm, void* stream) {
  ug::clear_error();
  ug_status st = check_plan(p, "ug_rope2d");
  if (st != UG_OK) return st;
  if (!q_perm || !k_perm) return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_rope2d: NULL tensor");
  if (!aligned16(q_perm) || !aligned16(k_perm))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_rope2d: tensors must be 16-byte aligned");
  if (overlap(q_perm, k_perm, tensor_bytes(p)))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_rope2d: q and k overlap");
  if (current_device() != p->device)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_rope2d: current device is not the plan's device");
  const int64_t rows = p->N + p->Nlr;
  if (rows == 0) return UG_OK;
  const int E = p->d.dtype == UG_BF16 ? 8 : 4;
  const int64_t units = int64_t(p->d.heads) * p->d.head_dim / E;
  const int64_t total = rows * units;
  const dim3 grid(unsigned((total + kRopeThreads - 1) / kRopeThreads), unsigned(p->d.batch));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float2* cs = reinterpret_cast<const float2*>(p->d_rope);
  const int32_t lr_w = std::max(p->d.lr_w, 1);
  if (p->d.dtype == UG_BF16)
    hipLaunchKernelGGL(rope2d_kernel<__bf16>, grid, dim3(kRopeThreads), 0, s, static_cast<__bf16*>(q_perm),
                       static_cast<__bf16*>(k_perm), int32_t(p->L), int32_t(p->T), int32_t(p->N), p->d.hr_w, lr_w,
                       p->d.rho, p->d.heads, p->d.head_dim, p->d_perm, cs);
  else
    hipLaunchKernelGGL(rope2d_kernel<float>, grid, dim3(kRopeThreads), 0, s, static_cast<float*>(q_perm),
                       static_cast<float*>(k_perm), int32_t(p->L), int32_t(p->T), int32_t(p->N), p->d.hr_w, lr_w,
                       p->d.rho, p->d.heads, p->d.head_dim, p->d_perm, cs);
  return launch_status("ug_rope2d");
}

ug_status ug_attn_fwd(ug_plan_t p, const void* q, const void* k, const void* v, void* o, void* workspace,
                      void* stream) {
  ug::clear_error();
  (void)workspace;
  ug_status st = check_plan(p, "ug_attn_fwd");
  if (st != UG_OK) return st;
  if (!q || !k || !v || !o) return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_attn_fwd: NULL tensor");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_attn_fwd: tensors must be 16-byte aligned");
  const int64_t n = tensor_bytes(p);
  if (overlap(o, q, n) || overlap(o, k, n) || overlap(o, v, n))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_attn_fwd: o overlaps q, k or v");
  if (current_device() != p->device)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_attn_fwd: current device is not the plan's device");
  if (p->blocks.empty()) return UG_OK;
  AttnParams ap{};
  ap.q = q;
  ap.k = k;
  ap.v = v;
  ap.o = o;
  ap.row_stride = int64_t(p->d.heads) * p->d.head_dim;
  ap.batch_stride = p->L * ap.row_stride;
  ap.heads = p->d.heads;
  ap.tasks = p->d_tasks;
  ap.ranges = p->d_ranges;
  ap.blocks = p->d_blocks;
  ap.scale_log2 = float(1.4426950408889634 / std::sqrt(double(p->d.head_dim)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = p->d.dtype == UG_BF16;
  if (bf && p->d.head_dim == 128)
    launch_attn<__bf16, 128>(p, ap, s);
  else if (bf && p->d.head_dim == 64)
    launch_attn<__bf16, 64>(p, ap, s);
  else if (!bf && p->d.head_dim == 128)
    launch_attn<float, 128>(p, ap, s);
  else
    launch_attn<float, 64>(p, ap, s);
  return launch_status("ug_attn_fwd");
}

}  // extern "C"
