// gfx950 kernel of the guidance-weighted warm start and its C-ABI entry point
// ug_warm_start.
//
// Method: UltraGen starts HR sampling at an intermediate time t instead of
// from pure noise ("UltraGen: Efficient Ultra-High-Resolution Image
// Generation with Hierarchical Local Attention", papernotes.org notes,
// 关键设计 4; gist.science summary, section 2.C): the LR latent is upsampled
// and sharpened into a reference Y, and the HR start latent is
//   X_hr = alpha * X_T + (1 - alpha) * Y,   alpha = t / T,
// with X_T Gaussian noise (an input).  Operators (the pages name them only):
//   U = bilinear interpolation, LR sample (m, n) at HR (rho*m, rho*n), the
//       last sample's value past the last LR row / column;
//   Y = U + s * (U - B*U), B the 3x3 binomial blur [1 2 1]/4 x [1 2 1]/4
//       with replicated edges, s the sharpening strength.
// Both operators are linear, so Y at an HR pixel is a 3x3 stencil on the LR
// samples: per axis, the weights of the plain interpolation (wc) and of the
// blurred one (wb) over three consecutive LR rows (columns), and
//   Y = sum_ij ((1 + s) wc_y[i] wc_x[j] - s wb_y[i] wb_x[j]) X_lr[y0+i][x0+j].
// HBM-bound: every noise and output byte moves once; the LR samples a tile
// needs are read once into LDS, and each thread forms the stencil
// separably (see the kernel).
#include "common.hpp"

#include <cmath>
#include <type_traits>

namespace {

using namespace ug::dev;
using ug::host::aligned16;
using ug::host::current_device;
using ug::host::launch_status;
using ug::host::overlap_ranges;

constexpr int kWarmThreads = 256;

// Weights of one axis at HR coordinate r: LR indices base .. base+2 (some
// may be clamped duplicates with zero weight).
struct AxisWeights {
  int base;
  float wc[3];  // plain bilinear interpolation at r
  float wb[3];  // [1 2 1]/4 blur of the interpolation over r-1, r, r+1 (clamped)
};

__device__ __forceinline__ AxisWeights axis_weights(int r, int n_hr, int n_lr, int rho) {
  AxisWeights a;
  a.base = min(max(r - 1, 0) / rho, n_lr - 1);
#pragma unroll
  for (int i = 0; i < 3; ++i) a.wc[i] = a.wb[i] = 0.f;
#pragma unroll
  for (int d = -1; d <= 1; ++d) {
    const int rr = min(max(r + d, 0), n_hr - 1);
    const int y0 = min(rr / rho, n_lr - 1);
    const float f = y0 < n_lr - 1 ? float(rr - y0 * rho) / float(rho) : 0.f;
    const int i0 = y0 - a.base;  // 0 .. 2, and i0 + 1 <= 2 whenever f > 0
    const float b = d == 0 ? 0.5f : 0.25f;
#pragma unroll
    for (int k = 0; k < 3; ++k) {  // selects, not a runtime array index
      const float wk = (k == i0 ? 1.f - f : 0.f) + (k == i0 + 1 ? f : 0.f);
      a.wb[k] += b * wk;
      if (d == 0) a.wc[k] += wk;
    }
  }
  return a;
}

template <typename T>
__device__ __forceinline__ void load_f32(const T* p, float (&x)[16 / sizeof(T)]) {
  constexpr int E = 16 / sizeof(T);
  if constexpr (std::is_same<T, float>::value) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x, x[1] = v.y, x[2] = v.z, x[3] = v.w;
  } else {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = float(v[e]);
  }
}

// One workgroup per HR tile of kTileH x kTileW pixels and a block of up to
// kVecBlock 16-byte channel vectors; thread (column, vector) produces the
// tile's kTileH pixels of its column, so that noise and output rows are
// contiguous across the workgroup.  The stencil is separable: with
//   Hc[m] = sum_j wc_x[j] X[m][x0+j],  Hb[m] = sum_j wb_x[j] X[m][x0+j]
// (the column passes of LR row m), the pixel's value is
//   sum_i (1 + s) wc_y[i] Hc[y0+i] - s wb_y[i] Hb[y0+i].
// The row weights also carry the blend's factor 1 - alpha, so the output is
// one more FMA with alpha and the noise.  A thread keeps the column passes of three consecutive LR rows in
// registers and slides them down as the tile's rows move to the next LR
// row, so each LR sample is converted and weighted once per thread.
constexpr int kTileH = 8, kVecBlock = 8, kTileW = kWarmThreads / kVecBlock;

__host__ __device__ constexpr int lr_span(int tile, int rho) { return (tile + 1) / rho + 3; }

struct RowWeights {  // one HR row: LR rows base .. base+2 with (1 - alpha)(1 + s) wc and (1 - alpha) s wb
  int base;
  float ca[3], cb[3];
};

template <typename T>
__global__ __launch_bounds__(kWarmThreads) void warm_start_kernel(const T* __restrict__ x_lr, const T* noise,
                                                                 T* x_hr,  // may be noise itself
                                                                 int32_t H, int32_t W, int32_t h, int32_t w,
                                                                 int32_t C, int32_t rho, float alpha, float s) {
  constexpr int E = 16 / sizeof(T);
  extern __shared__ __attribute__((aligned(16))) char warm_smem[];
  __shared__ RowWeights s_ay[kTileH];
  __shared__ AxisWeights s_ax[kTileW];

  const int32_t vpp = C / E;                             // vectors per pixel
  const int32_t nvb = (vpp + kVecBlock - 1) / kVecBlock;  // vector blocks
  const int32_t tiles_x = (W + kTileW - 1) / kTileW;
  int32_t t = blockIdx.x;
  const int32_t vb = t % nvb;
  t /= nvb;
  const int32_t r0 = (t / tiles_x) * kTileH, c0 = (t % tiles_x) * kTileW;
  const int32_t v0 = vb * kVecBlock, nv = min(kVecBlock, vpp - v0);
  const int64_t b = blockIdx.y;
  const int tid = threadIdx.x;
  const int v = tid % kVecBlock, cl = tid / kVecBlock;
  const int32_t c = c0 + cl;
  const bool col_ok = v < nv && c < W;

  // The thread's noise vectors first, so their loads are in flight while the
  // LR patch is staged (rows past a ragged edge load vector 0, store nothing).
  const u32x4* nzv = reinterpret_cast<const u32x4*>(noise) + b * int64_t(H) * W * vpp;
  u32x4* outv = reinterpret_cast<u32x4*>(x_hr) + b * int64_t(H) * W * vpp;
  const int64_t g0 = (int64_t(r0) * W + c) * vpp + v0 + v;
  const int64_t row_step = int64_t(W) * vpp;
  u32x4 nz[kTileH];
#pragma unroll
  for (int k = 0; k < kTileH; ++k) {
    const bool ok = col_ok && r0 + k < H;
    nz[k] = __builtin_nontemporal_load(nzv + (ok ? g0 + k * row_step : 0));
  }

  // LR rows [y_lo, y_hi] and columns [x_lo, x_hi] the tile's stencils touch
  const int32_t y_lo = min(max(r0 - 1, 0) / rho, h - 1);
  const int32_t y_hi = min(min(r0 + kTileH, H - 1) / rho + 1, h - 1);
  const int32_t x_lo = min(max(c0 - 1, 0) / rho, w - 1);
  const int32_t x_hi = min(min(c0 + kTileW, W - 1) / rho + 1, w - 1);
  const int32_t ny = y_hi - y_lo + 1, nx = x_hi - x_lo + 1;

  u32x4* const lds = reinterpret_cast<u32x4*>(warm_smem);  // [ny][nx][nv]
  const u32x4* lr = reinterpret_cast<const u32x4*>(x_lr) + b * int64_t(h) * w * vpp;
  for (int32_t i = tid; i < ny * nx * nv; i += kWarmThreads) {
    const int32_t vv = i % nv, px = i / nv;
    const int32_t yy = y_lo + px / nx, xx = x_lo + px % nx;
    lds[i] = lr[(int64_t(yy) * w + xx) * vpp + v0 + vv];
  }
  if (tid < kTileH) {
    const AxisWeights a = axis_weights(min(r0 + tid, H - 1), H, h, rho);
    RowWeights rw;
    rw.base = a.base;
#pragma unroll
    for (int i = 0; i < 3; ++i) rw.ca[i] = (1.f - alpha) * (1.f + s) * a.wc[i], rw.cb[i] = (1.f - alpha) * s * a.wb[i];
    s_ay[tid] = rw;
  }
  if (tid >= 64 && tid < 64 + kTileW) s_ax[tid - 64] = axis_weights(min(c0 + tid - 64, W - 1), W, w, rho);
  __syncthreads();

  const AxisWeights ax = s_ax[cl];
  int32_t lxo[3];
#pragma unroll
  // Every tap with a nonzero weight lies in the staged patch; a third tap
  // that does not (zero weight) is clamped into it, so it reads a staged
  // (finite) sample rather than whatever the LDS held before.  Threads past
  // the block's vectors (nothing to store) read the last staged vector.
  for (int j = 0; j < 3; ++j) lxo[j] = (min(ax.base + j, x_hi) - x_lo) * nv + min(v, nv - 1);
  // column passes of LR row y (clamped into the patch) into hc, hb
  auto column_pass = [&](int32_t y, float (&hc)[E], float (&hb)[E]) {
    const int32_t lrow = (min(y, y_hi) - y_lo) * nx * nv;
    UG_CHECK(lrow >= 0 && lrow + lxo[0] < ny * nx * nv && lrow + lxo[2] < ny * nx * nv && lxo[0] >= 0, 5);
#pragma unroll
    for (int e = 0; e < E; ++e) hc[e] = hb[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const u32x4 xv = lds[lrow + lxo[j]];
      float x[E];
      load_f32<T>(reinterpret_cast<const T*>(&xv), x);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        hc[e] = fmaf(ax.wc[j], x[e], hc[e]);
        hb[e] = fmaf(ax.wb[j], x[e], hb[e]);
      }
    }
  };
  // Output row k of the tile from the column passes of its three LR rows.
  auto emit_row = [&](int k, const RowWeights& ay, const float (&c0)[E], const float (&c1)[E], const float (&c2)[E],
                      const float (&b0)[E], const float (&b1)[E], const float (&b2)[E]) {
    float nf[E];
    load_f32<T>(reinterpret_cast<const T*>(&nz[k]), nf);
    float o32[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float acc = ay.ca[0] * c0[e];
      acc = fmaf(ay.ca[1], c1[e], acc);
      acc = fmaf(ay.ca[2], c2[e], acc);
      acc = fmaf(-ay.cb[0], b0[e], acc);
      acc = fmaf(-ay.cb[1], b1[e], acc);
      acc = fmaf(-ay.cb[2], b2[e], acc);
      o32[e] = fmaf(alpha, nf[e], acc);  // acc carries the factor 1 - alpha
    }
    u32x4 out;
    if constexpr (std::is_same<T, float>::value) {
      float* o = reinterpret_cast<float*>(&out);
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = o32[e];
    } else {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = __bf16(o32[e]);
      out = *reinterpret_cast<u32x4*>(&o);
    }
    UG_CHECK(!(col_ok && r0 + k < H) || (g0 + k * row_step >= 0 && g0 + k * row_step < int64_t(H) * W * vpp), 5);
    if (col_ok && r0 + k < H) __builtin_nontemporal_store(out, outv + g0 + k * row_step);
  };
  // Interior tiles at rho 4: the rows' LR bases are b-1 (row 0), b (rows 1-4)
  // and b+1 (rows 5-7) with b = r0 / 4, so the three sets of column passes
  // rotate at compile time (row b+2's pass overwrites row b-1's set after
  // row 0, row b+3's overwrites row b's after row 4) instead of sliding down
  // with moves as in the general path below.
  const bool fixed4 = rho == 4 && r0 >= kTileH && r0 + kTileH <= H && (r0 + kTileH - 2) / 4 <= h - 1;
  if (fixed4) {  // uniform
    const int32_t b4 = r0 / 4;
    float c0[E], c1[E], c2[E], d0[E], d1[E], d2[E];
    column_pass(b4 - 1, c0, d0);
    column_pass(b4, c1, d1);
    column_pass(b4 + 1, c2, d2);
#pragma unroll
    for (int k = 0; k < kTileH; ++k) {
      const RowWeights ay = s_ay[k];
      if (k == 1) column_pass(b4 + 2, c0, d0);
      if (k == 5) column_pass(b4 + 3, c1, d1);
      UG_CHECK(ay.base == b4 - 1 + (k == 0 ? 0 : k <= 4 ? 1 : 2), 5);
      if (k == 0) emit_row(k, ay, c0, c1, c2, d0, d1, d2);
      else if (k <= 4) emit_row(k, ay, c1, c2, c0, d1, d2, d0);
      else emit_row(k, ay, c2, c0, c1, d2, d0, d1);
    }
    return;
  }
  float hc[3][E], hb[3][E];
  int32_t held = s_ay[0].base;  // LR row of hc[0] / hb[0] (uniform)
#pragma unroll
  for (int i = 0; i < 3; ++i) column_pass(held + i, hc[i], hb[i]);

#pragma unroll
  for (int k = 0; k < kTileH; ++k) {
    const RowWeights ay = s_ay[k];
    while (held < ay.base) {  // uniform; at most one step per row for rho >= 1
#pragma unroll
      for (int e = 0; e < E; ++e) {
        hc[0][e] = hc[1][e], hb[0][e] = hb[1][e];
        hc[1][e] = hc[2][e], hb[1][e] = hb[2][e];
      }
      ++held;
      column_pass(held + 2, hc[2], hb[2]);
    }
    emit_row(k, ay, hc[0], hc[1], hc[2], hb[0], hb[1], hb[2]);
  }
}

}  // namespace

extern "C" {

ug_status ug_warm_start(const ug_warm_desc* d, const void* x_lr, const void* noise, void* x_hr, void* stream) {
  const char* fn = "ug_warm_start";
  ug::clear_error();
  if (!d) return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_warm_start: desc is NULL");
  if (d->dtype != UG_F32 && d->dtype != UG_BF16)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_warm_start: dtype must be UG_F32 or UG_BF16");
  const int E = d->dtype == UG_BF16 ? 8 : 4;
  if (d->batch < 1 || d->hr_h < 1 || d->hr_w < 1 || d->lr_h < 1 || d->lr_w < 1 || d->rho < 1)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_warm_start: batch, grids and rho must be positive");
  if (d->channels < 1 || d->channels % E != 0)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_warm_start: channels must be a positive multiple of " +
                                                 std::to_string(E) + " (one 16-byte vector)");
  if (!std::isfinite(d->alpha) || d->alpha < 0.f || d->alpha > 1.f)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_warm_start: alpha must be in [0, 1]");
  if (!std::isfinite(d->sharpen) || d->sharpen < 0.f)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_warm_start: sharpen must be finite and >= 0");
  if (!x_lr || !noise || !x_hr || !aligned16(x_lr) || !aligned16(noise) || !aligned16(x_hr))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_warm_start: tensors must be non-NULL and 16-byte aligned");
  const int64_t esize = d->dtype == UG_BF16 ? 2 : 4;
  const int64_t n_hr = int64_t(d->batch) * d->hr_h * d->hr_w * d->channels * esize;
  const int64_t n_lr = int64_t(d->batch) * d->lr_h * d->lr_w * d->channels * esize;
  if (overlap_ranges(x_hr, n_hr, x_lr, n_lr))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_warm_start: x_hr overlaps x_lr");
  if (x_hr != noise && overlap_ranges(x_hr, n_hr, noise, n_hr))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_warm_start: x_hr partly overlaps noise (only x_hr == noise is allowed)");
  if (current_device() < 0) return ug::fail(UG_ERR_HIP, "ug_warm_start: no HIP device is current");
  const int32_t vpp = d->channels / E;
  const int64_t tiles = int64_t((d->hr_h + kTileH - 1) / kTileH) * ((d->hr_w + kTileW - 1) / kTileW) *
                        ((vpp + kVecBlock - 1) / kVecBlock);
  if (tiles > 0x7fffffff || d->batch > 65535)
    return ug::fail(UG_ERR_UNSUPPORTED, "ug_warm_start: tensor too large for one launch");
  const size_t lds = size_t(lr_span(kTileH, d->rho)) * lr_span(kTileW, d->rho) * kVecBlock * 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(tiles), unsigned(d->batch));
  if (d->dtype == UG_BF16)
    hipLaunchKernelGGL(warm_start_kernel<__bf16>, grid, dim3(kWarmThreads), lds, s, static_cast<const __bf16*>(x_lr),
                       static_cast<const __bf16*>(noise), static_cast<__bf16*>(x_hr), d->hr_h, d->hr_w, d->lr_h,
                       d->lr_w, d->channels, d->rho, d->alpha, d->sharpen);
  else
    hipLaunchKernelGGL(warm_start_kernel<float>, grid, dim3(kWarmThreads), lds, s, static_cast<const float*>(x_lr),
                       static_cast<const float*>(noise), static_cast<float*>(x_hr), d->hr_h, d->hr_w, d->lr_h,
                       d->lr_w, d->channels, d->rho, d->alpha, d->sharpen);
  return launch_status(fn);
}

}  // extern "C"

UG_BOUNDS_ACCESSOR(ug_debug_bounds_warm)
