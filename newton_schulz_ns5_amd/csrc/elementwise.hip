// Bandwidth-bound kernels of the step: momentum / load with orientation and
// Frobenius-norm partials, the norm finalize, NorMuon row statistics, the
// NorMuon norm-preserving factor, and the weight update.
//
// All reductions run in a fixed order that depends only on the matrix shape
// (per-thread sums in index order, wave64 xor butterflies, then the four
// waves of a workgroup in index order; per-matrix partials summed the same
// way), so every result is deterministic and independent of the batch.
#include "muon_internal.h"
#include "device_util.h"
#include "muon_mi355x.h"

namespace muon {
namespace {

__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Load 16 consecutive elements [c, c+16) of a row, zero beyond `valid`.
__device__ __forceinline__ void load16(const void* row, int c, int valid, bool bf, bool vec, float* out) {
  if (vec && c + 16 <= valid) {
    if (bf) {
      const u32x4* p = (const u32x4*)((const uint16_t*)row + c);
      const u32x4 a = p[0], b = p[1];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        out[2 * w] = __uint_as_float(a[w] << 16);
        out[2 * w + 1] = __uint_as_float(a[w] & 0xffff0000u);
        out[8 + 2 * w] = __uint_as_float(b[w] << 16);
        out[8 + 2 * w + 1] = __uint_as_float(b[w] & 0xffff0000u);
      }
    } else {
      const f32x4* p = (const f32x4*)((const float*)row + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 t = p[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) out[4 * q + e] = t[e];
      }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) out[e] = (c + e < valid) ? load_elem(row, c + e, bf) : 0.f;
}

// Load 8 consecutive elements [0, 8) of a row, zero beyond `valid`.
__device__ __forceinline__ void load8(const void* row, int valid, bool bf, bool vec, float* out) {
  if (vec && valid >= 8) {
    if (bf) {
      const u32x4 a = *(const u32x4*)row;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        out[2 * w] = __uint_as_float(a[w] << 16);
        out[2 * w + 1] = __uint_as_float(a[w] & 0xffff0000u);
      }
    } else {
      const f32x4 a = ((const f32x4*)row)[0], b = ((const f32x4*)row)[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) { out[e] = a[e]; out[4 + e] = b[e]; }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = e < valid ? load_elem(row, e, bf) : 0.f;
}

// Store v[0 .. 8) (all eight with vector stores when `vec`, else the first
// `valid`).
__device__ __forceinline__ void store8v(void* row, int valid, bool bf, bool vec, const float* v) {
  if (vec && valid >= 8) {
    if (bf) {
      u32x4 a;
#pragma unroll
      for (int w = 0; w < 4; ++w) a[w] = pack_bf2(v[2 * w], v[2 * w + 1]);
      *(u32x4*)row = a;
    } else {
      f32x4 a, b;
#pragma unroll
      for (int e = 0; e < 4; ++e) { a[e] = v[e]; b[e] = v[4 + e]; }
      ((f32x4*)row)[0] = a;
      ((f32x4*)row)[1] = b;
    }
    return;
  }
  for (int e = 0; e < 8 && e < valid; ++e) store_elem(row, e, v[e], bf);
}

// One 64 x 64 tile of the oriented, padded X0 per workgroup.
//   mode 0: U = x (muon_ns_batched input)
//   mode 1: M <- mu M + G;  U = G + mu M  (or U = M without Nesterov)
// Writes U (rounded to the X dtype) at its oriented position, zeros in the
// padding, and the tile's sum of U^2 (from the fp32 U) to partial[]; with
// no_x (a bf16 input the iterations read in place) the partials only.
// Thread -> rows tid / 8 and tid / 8 + 32 of the tile, 8 consecutive columns
// each: eight lanes cover one 64-element row segment, so every wave access
// is whole 128-byte lines (bf16).  The tile is staged in LDS for the
// transposed write of a tall matrix.
// One launch covers the problems of a PrepGroup: the grid's z index picks the
// problem and its matrix, and a problem smaller than the grid's x/y extent
// leaves the rest of the grid idle.
__global__ __launch_bounds__(256) void prep_kernel(const PrepGroup grp) {
  __shared__ float T[64][65];
  __shared__ float red[4];
  int pi = 0;
  while (pi + 1 < grp.nprob && (int)blockIdx.z >= grp.zstart[pi + 1]) ++pi;
  const PrepParams& p = grp.prob[pi];
  const int tiles_x = p.np / 64, tiles_y = p.mp / 64;
  if ((int)blockIdx.x >= tiles_x || (int)blockIdx.y >= tiles_y) return;
  const int tid = threadIdx.x;
  const int bz = (int)blockIdx.z - grp.zstart[pi];
  const int oi0 = blockIdx.y * 64, oj0 = blockIdx.x * 64;
  const int pr0 = p.tall ? oj0 : oi0, pc0 = p.tall ? oi0 : oj0;
  const int c0 = (tid & 7) * 8;
  const int gc = pc0 + c0;
  const bool src_bf = p.src_dtype == MUON_BF16;
  float s = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (tid >> 3) + 32 * h;
    const int gr = pr0 + r;
    float u[8];
    if (p.mode == 0) {
      const void* row = (const uint8_t*)p.x +
                        ((int64_t)bz * p.x_bs + (int64_t)gr * p.x_rs + gc) * (src_bf ? 2 : 4);
      const int valid = gr < p.rows ? p.cols - gc : 0;
      const bool vec = ((p.x_rs | p.x_bs) & 7) == 0 && ((uintptr_t)p.x & 15) == 0;
      float tmp[8];
      if (valid > 0) load8(row, valid, src_bf, vec, tmp);
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = valid > 0 ? tmp[e] : 0.f;
    } else {
      const int par = bz / p.heads, hd = bz - par * p.heads;
      const bool mom_bf = p.mom_dtype == MUON_BF16;
      const int64_t off = (int64_t)(hd * p.rows + gr) * p.param_cols + gc;
      const int valid = gr < p.rows ? p.cols - gc : 0;
      const bool vec = (p.param_cols & 7) == 0;
      float g[8], m[8];
      if (valid > 0) {
        load8((const uint8_t*)p.grad[par] + off * (src_bf ? 2 : 4), valid, src_bf, vec, g);
        load8((const uint8_t*)p.mom[par] + off * (mom_bf ? 2 : 4), valid, mom_bf, vec, m);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e < valid) {
          const float mn = p.mu * m[e] + g[e];
          u[e] = p.nesterov ? g[e] + p.mu * mn : mn;
          m[e] = mn;
        } else {
          u[e] = 0.f;
        }
      }
      if (valid > 0) store8v((uint8_t*)p.mom[par] + off * (mom_bf ? 2 : 4), valid, mom_bf, vec, m);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s += u[e] * u[e];
      T[r][c0 + e] = u[e];
    }
  }
  if (!p.no_x) {
    __syncthreads();
    // Oriented write: X[oi0 + orow][oj0 + c0 .. +8].
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int orow = (tid >> 3) + 32 * h;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = p.tall ? T[c0 + e][orow] : T[orow][c0 + e];
      const int64_t xoff = (int64_t)bz * p.X_bs + (int64_t)(oi0 + orow) * p.np + oj0 + c0;
      store8v((uint8_t*)p.X + xoff * (p.x_bf16 ? 2 : 4), 8, p.x_bf16, true, v);
    }
  }
  const float tot = block_sum(s, red);
  if (tid == 0) p.partial[(int64_t)bz * (tiles_x * tiles_y) + blockIdx.y * tiles_x + blockIdx.x] = tot;
}

// rs[b] = 1 / (sqrt(sum of the matrix's tile partials) + eps).  A sum that
// is not finite (an input whose squared Frobenius norm exceeds the fp32
// range, or a NaN in it) gives rs = NaN, so the output is NaN rather than a
// silently zero matrix.
__global__ __launch_bounds__(256) void norm_kernel(const NormGroup grp) {
  __shared__ float red[4];
  int pi = 0;
  while (pi + 1 < grp.nprob && (int)blockIdx.x >= grp.start[pi + 1]) ++pi;
  const NormParams& p = grp.prob[pi];
  const int b = (int)blockIdx.x - grp.start[pi];
  const float* src = p.partial + (int64_t)b * p.tiles;
  float s = 0.f;
  int i = threadIdx.x;
  // Eight loads in flight per thread (a matrix has up to tens of thousands of
  // partials); they are still added one by one in index order.
  for (; i + 7 * 256 < p.tiles; i += 8 * 256) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[i + 256 * k];
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[k];
  }
  for (; i < p.tiles; i += 256) s += src[i];
  const float tot = block_sum(s, red);
  if (threadIdx.x == 0) p.rs[b] = __builtin_isfinite(tot) ? 1.f / (sqrtf(tot) + p.eps) : __builtin_nanf("");
}

// Split-K Gram: A = bf16(rs^2 * (part_0 + part_1 + ...)), the chunks added in
// order.  Thread -> 8 consecutive elements of one row of the mp x mp matrix.
__global__ __launch_bounds__(256) void split_sum_kernel(const SplitSumParams p) {
  const int b = blockIdx.y;
  const int64_t mm = (int64_t)p.mp * p.mp;
  const int64_t e8 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  const float* src = p.part + (int64_t)b * p.ksplit * mm + e8;
  f32x4 s0 = *(const f32x4*)src, s1 = *(const f32x4*)(src + 4);
  for (int k = 1; k < p.ksplit; ++k) {
    const f32x4 t0 = *(const f32x4*)(src + k * mm), t1 = *(const f32x4*)(src + k * mm + 4);
    s0 += t0;
    s1 += t1;
  }
  const float rsb = p.rs ? p.rs[b] : 1.f;
  const float alpha = rsb * rsb;
  u32x4 w;
  w[0] = pack_bf2(alpha * s0[0], alpha * s0[1]);
  w[1] = pack_bf2(alpha * s0[2], alpha * s0[3]);
  w[2] = pack_bf2(alpha * s1[0], alpha * s1[1]);
  w[3] = pack_bf2(alpha * s1[2], alpha * s1[3]);
  const int64_t i = e8 / p.mp, j = e8 - i * p.mp;
  *(u32x4*)((uint16_t*)p.A + (int64_t)b * p.a_bs + i * p.lda + j) = w;
}

// NorMuon row statistics: one wave64 per row.  Lane l sums the squares of
// elements 512 t + 8 l + e (t = 0, 1, ...; e = 0..7) in that order.
__global__ __launch_bounds__(256) void rowstat_kernel(const RowStatGroup grp) {
  int pi = 0;
  while (pi + 1 < grp.nprob && (int)blockIdx.y >= grp.start[pi + 1]) ++pi;
  const RowStatParams& p = grp.prob[pi];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = (int)blockIdx.y - grp.start[pi];
  const int r = blockIdx.x * 4 + wave;
  if (r >= p.rows) return;
  const bool bf = p.o_dtype == MUON_BF16;
  const uint8_t* row = (const uint8_t*)p.O + ((int64_t)b * p.o_bs + (int64_t)r * p.o_rs) * (bf ? 2 : 4);
  const bool vec = ((p.o_bs | p.o_rs) & 7) == 0 && ((uintptr_t)p.O & 15) == 0;
  float s = 0.f;
  int c = lane * 8;
  if (vec) {
    // Four chunks in flight per lane; their squares are still added chunk by
    // chunk in column order, as in the loop below.
    for (; c + 3 * 512 + 8 <= p.cols; c += 4 * 512) {
      float x[4][8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int ck = c + 512 * k;
        if (bf) {
          const u32x4 a = *(const u32x4*)(row + (int64_t)ck * 2);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            x[k][2 * w] = __uint_as_float(a[w] << 16);
            x[k][2 * w + 1] = __uint_as_float(a[w] & 0xffff0000u);
          }
        } else {
          const f32x4 a = *(const f32x4*)(row + (int64_t)ck * 4), b2 = *(const f32x4*)(row + (int64_t)ck * 4 + 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) { x[k][e] = a[e]; x[k][4 + e] = b2[e]; }
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) s += x[k][e] * x[k][e];
    }
  }
  for (; c < p.cols; c += 512) {
    float x[8];
    if (vec && c + 8 <= p.cols) {
      if (bf) {
        const u32x4 a = *(const u32x4*)(row + (int64_t)c * 2);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          x[2 * w] = __uint_as_float(a[w] << 16);
          x[2 * w + 1] = __uint_as_float(a[w] & 0xffff0000u);
        }
      } else {
        const f32x4 a = *(const f32x4*)(row + (int64_t)c * 4), b2 = *(const f32x4*)(row + (int64_t)c * 4 + 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b2[e]; }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (c + e < p.cols) ? load_elem(row, c + e, bf) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s += x[e] * x[e];
  }
  s = wave_sum(s);
  if (lane == 0) {
    const float ms = s / (float)p.cols;
    float* v = p.v_base ? p.v_base + (int64_t)b * p.v_bs : p.v_tab[b];
    const float vn = p.beta2 * v[r] + (1.f - p.beta2) * ms;
    v[r] = vn;
    const float d = 1.f / (sqrtf(vn) + p.eps);
    const int64_t o = (int64_t)b * p.rows + r;
    p.d[o] = d;
    p.ms[o] = ms;
    p.q[o] = d * d * ms;
  }
}

// rho[b] = ||O||_F / ||diag(d) O||_F = sqrt(sum ms / sum d^2 ms); 0 when the
// normalized matrix is zero.
__global__ __launch_bounds__(256) void rho_kernel(const RhoGroup grp) {
  __shared__ float red[4];
  int pi = 0;
  while (pi + 1 < grp.nprob && (int)blockIdx.x >= grp.start[pi + 1]) ++pi;
  const RhoParams& p = grp.prob[pi];
  const int b = (int)blockIdx.x - grp.start[pi];
  const float* ms = p.ms + (int64_t)b * p.rows;
  const float* qq = p.q + (int64_t)b * p.rows;
  float a = 0.f, q = 0.f;
  int i = threadIdx.x;
  // Four rows of each in flight per thread, added one by one in row order.
  for (; i + 3 * 256 < p.rows; i += 4 * 256) {
    float va[4], vq[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      va[k] = ms[i + 256 * k];
      vq[k] = qq[i + 256 * k];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a += va[k];
      q += vq[k];
    }
  }
  for (; i < p.rows; i += 256) {
    a += ms[i];
    q += qq[i];
  }
  const float sa = block_sum(a, red);
  __syncthreads();
  const float sq = block_sum(q, red);
  if (threadIdx.x == 0) p.rho[b] = sq > 0.f ? sqrtf(sa / sq) : 0.f;
}

// One wave64 per row.  mode 0: W <- decay W - coef_r O (fp32 fused
// multiply-add, one rounding) and the optional bf16 copy; mode 1: O <- coef_r O.
__global__ __launch_bounds__(256) void apply_kernel(const ApplyGroup grp) {
  int pi = 0;
  while (pi + 1 < grp.nprob && (int)blockIdx.y >= grp.start[pi + 1]) ++pi;
  const ApplyParams& p = grp.prob[pi];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = (int)blockIdx.y - grp.start[pi];
  const int r = blockIdx.x * 4 + wave;
  if (r >= p.rows) return;
  const bool bf = p.o_dtype == MUON_BF16;
  uint8_t* orow = (uint8_t*)p.O + ((int64_t)b * p.o_bs + (int64_t)r * p.o_rs) * (bf ? 2 : 4);
  const float dr = p.d ? p.d[(int64_t)b * p.rows + r] : 1.f;
  const float rho = p.rho ? p.rho[b] : 1.f;
  if (p.mode == 1) {
    const float coef = rho * dr;
    for (int c = lane; c < p.cols; c += 64) store_elem(orow, c, coef * load_elem(orow, c, bf), bf);
    return;
  }
  const float coef = p.lr_eff * (rho * dr);
  float* w = p.w[b] + (int64_t)r * p.cols;
  uint16_t* wm = p.wm[b] ? (uint16_t*)p.wm[b] + (int64_t)r * p.cols : nullptr;
  if (p.vec) {
    // Two chunks per lane per step: both chunks' loads are issued before
    // either is stored (O and W are distinct buffers).
    int c = lane * 8;
    for (; c + 512 < p.cols; c += 1024) {
      float o[2][8];
      f32x4 w0[2], w1[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int ck = c + 512 * k;
        if (bf) {
          const u32x4 a = *(const u32x4*)(orow + (int64_t)ck * 2);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            o[k][2 * q] = __uint_as_float(a[q] << 16);
            o[k][2 * q + 1] = __uint_as_float(a[q] & 0xffff0000u);
          }
        } else {
          const f32x4 a = *(const f32x4*)(orow + (int64_t)ck * 4), b2 = *(const f32x4*)(orow + (int64_t)ck * 4 + 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) { o[k][e] = a[e]; o[k][4 + e] = b2[e]; }
        }
        w0[k] = *(const f32x4*)(w + ck);
        w1[k] = *(const f32x4*)(w + ck + 4);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int ck = c + 512 * k;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w0[k][e] = fmaf(-coef, o[k][e], p.decay * w0[k][e]);
          w1[k][e] = fmaf(-coef, o[k][4 + e], p.decay * w1[k][e]);
        }
        *(f32x4*)(w + ck) = w0[k];
        *(f32x4*)(w + ck + 4) = w1[k];
        if (wm) {
          u32x4 t;
          t[0] = pack_bf2(w0[k][0], w0[k][1]);
          t[1] = pack_bf2(w0[k][2], w0[k][3]);
          t[2] = pack_bf2(w1[k][0], w1[k][1]);
          t[3] = pack_bf2(w1[k][2], w1[k][3]);
          *(u32x4*)(wm + ck) = t;
        }
      }
    }
    for (; c < p.cols; c += 512) {
      float o[8];
      if (bf) {
        const u32x4 a = *(const u32x4*)(orow + (int64_t)c * 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o[2 * q] = __uint_as_float(a[q] << 16);
          o[2 * q + 1] = __uint_as_float(a[q] & 0xffff0000u);
        }
      } else {
        const f32x4 a = *(const f32x4*)(orow + (int64_t)c * 4), b2 = *(const f32x4*)(orow + (int64_t)c * 4 + 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) { o[e] = a[e]; o[4 + e] = b2[e]; }
      }
      f32x4 w0 = *(const f32x4*)(w + c), w1 = *(const f32x4*)(w + c + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = fmaf(-coef, o[e], p.decay * w0[e]);
        w1[e] = fmaf(-coef, o[4 + e], p.decay * w1[e]);
      }
      *(f32x4*)(w + c) = w0;
      *(f32x4*)(w + c + 4) = w1;
      if (wm) {
        u32x4 t;
        t[0] = pack_bf2(w0[0], w0[1]);
        t[1] = pack_bf2(w0[2], w0[3]);
        t[2] = pack_bf2(w1[0], w1[1]);
        t[3] = pack_bf2(w1[2], w1[3]);
        *(u32x4*)(wm + c) = t;
      }
    }
  } else {
    for (int c = lane; c < p.cols; c += 64) {
      const float nw = fmaf(-coef, load_elem(orow, c, bf), p.decay * w[c]);
      w[c] = nw;
      if (wm) wm[c] = f2bf(nw);
    }
  }
}

}  // namespace

hipError_t launch_prep_group(const PrepGroup& g, hipStream_t s) {
  if (g.nprob < 1 || g.nprob > kMaxPrep || g.zstart[0] != 0) return hipErrorInvalidValue;
  int gx = 0, gy = 0;
  for (int i = 0; i < g.nprob; ++i) {
    const PrepParams& p = g.prob[i];
    if (g.zstart[i + 1] < g.zstart[i] || p.np % kPrepTile || p.mp % kPrepTile) return hipErrorInvalidValue;
    gx = p.np / kPrepTile > gx ? p.np / kPrepTile : gx;
    gy = p.mp / kPrepTile > gy ? p.mp / kPrepTile : gy;
  }
  const int gz = g.zstart[g.nprob];
  if (gz <= 0 || gx <= 0 || gy <= 0) return hipSuccess;
  if (gz > 65535 || gy > 65535) return hipErrorInvalidValue;
  return launch_kernel(prep_kernel, dim3(gx, gy, gz), g, s);
}

hipError_t launch_norm_group(const NormGroup& g, hipStream_t s) {
  if (g.nprob < 1 || g.nprob > kMaxNorm || g.start[0] != 0) return hipErrorInvalidValue;
  for (int i = 0; i < g.nprob; ++i)
    if (g.start[i + 1] < g.start[i] || g.prob[i].tiles < 1) return hipErrorInvalidValue;
  const int grid = g.start[g.nprob];
  if (grid <= 0) return hipSuccess;
  return launch_kernel(norm_kernel, dim3(grid), g, s);
}


hipError_t launch_split_sum(const SplitSumParams& p, int nb, hipStream_t s) {
  // mp is a multiple of 128, so mp^2 / 8 is a whole number of 256-thread blocks.
  if (nb <= 0) return hipSuccess;
  if (p.mp <= 0 || p.mp % 128 != 0 || p.lda % 8 != 0 || p.ksplit < 1) return hipErrorInvalidValue;
  return launch_kernel(split_sum_kernel, dim3((unsigned)((int64_t)p.mp * p.mp / 8 / 256), nb), p, s);
}

// Grids of the grouped NorMuon / update launches: problem i owns grid y (or,
// for rho, x) indices start[i] .. start[i + 1] - 1, one per matrix (at most
// 65535 in all for y); the row extent is the largest problem's.
template <typename G>
static bool group_ok(const G& g, int kmax) {
  if (g.nprob < 1 || g.nprob > kmax || g.start[0] != 0) return false;
  for (int i = 0; i < g.nprob; ++i)
    if (g.start[i + 1] < g.start[i]) return false;
  return true;
}

hipError_t launch_rowstat_group(const RowStatGroup& g, hipStream_t s) {
  if (!group_ok(g, kMaxRowStat)) return hipErrorInvalidValue;
  int rows = 0;
  for (int i = 0; i < g.nprob; ++i) rows = g.prob[i].rows > rows ? g.prob[i].rows : rows;
  const int nb = g.start[g.nprob];
  if (nb <= 0 || rows <= 0) return hipSuccess;
  if (nb > 65535) return hipErrorInvalidValue;
  return launch_kernel(rowstat_kernel, dim3((rows + 3) / 4, nb), g, s);
}

hipError_t launch_rho_group(const RhoGroup& g, hipStream_t s) {
  if (!group_ok(g, kMaxRho)) return hipErrorInvalidValue;
  const int nb = g.start[g.nprob];
  if (nb <= 0) return hipSuccess;
  return launch_kernel(rho_kernel, dim3(nb), g, s);
}

hipError_t launch_apply_group(const ApplyGroup& g, hipStream_t s) {
  if (!group_ok(g, kMaxApply)) return hipErrorInvalidValue;
  int rows = 0;
  for (int i = 0; i < g.nprob; ++i) rows = g.prob[i].rows > rows ? g.prob[i].rows : rows;
  const int nb = g.start[g.nprob];
  if (nb <= 0 || rows <= 0) return hipSuccess;
  if (nb > 65535) return hipErrorInvalidValue;
  return launch_kernel(apply_kernel, dim3((rows + 3) / 4, nb), g, s);
}

hipError_t launch_rowstat(const RowStatParams& p, int nb, hipStream_t s) {
  if (nb <= 0 || p.rows <= 0) return hipSuccess;
  RowStatGroup g{};
  g.prob[0] = p;
  g.start[1] = nb;
  g.nprob = 1;
  return launch_rowstat_group(g, s);
}

hipError_t launch_rho(const RhoParams& p, int nb, hipStream_t s) {
  if (nb <= 0) return hipSuccess;
  RhoGroup g{};
  g.prob[0] = p;
  g.start[1] = nb;
  g.nprob = 1;
  return launch_rho_group(g, s);
}

hipError_t launch_apply(const ApplyParams& p, int nb, hipStream_t s) {
  if (nb <= 0 || p.rows <= 0) return hipSuccess;
  ApplyGroup g{};
  g.prob[0] = p;
  g.start[1] = nb;
  g.nprob = 1;
  return launch_apply_group(g, s);
}

}  // namespace muon
