// Per-step kernels shared by the fp32 and bf16 paths: probe seeds, token validation, the
// probe-independent +-eps weight tables, per-model perturbed small tensors, the per-probe loss
// reduction, and the seed-regenerating CD-RGE update.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "philox.h"

namespace cdrge {

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// 4 x 4 exchange among the lanes 16, 32 and 48 apart (the four 16-lane rows of a wave):
// afterwards a, b, c, d in row w hold what rows 0, 1, 2, 3 held in register w (a for w = 0, ...,
// d for w = 3). Two v_permlane16_swap and two v_permlane32_swap; all 64 lanes must be active.
__device__ __forceinline__ void row_exchange(uint32_t& a, uint32_t& b, uint32_t& c, uint32_t& d) {
  const auto s01 = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  const auto s23 = __builtin_amdgcn_permlane16_swap(c, d, false, false);
  const auto t02 = __builtin_amdgcn_permlane32_swap(s01[0], s23[0], false, false);
  const auto t13 = __builtin_amdgcn_permlane32_swap(s01[1], s23[1], false, false);
  a = t02[0];
  b = t13[0];
  c = t02[1];
  d = t13[1];
}

// Nearest bf16 to x, ties to even; NaN stays a quiet NaN. (The carry of the rounding increment
// propagates into the exponent, so values past the largest bf16 become infinity.)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const bool nan = (u & 0x7fffffffu) > 0x7f800000u;
  return nan ? ((u >> 16) | 0x40u) : rounded;  // a select, not a branch
}

// A perturbed weight: w + s*eps with s in {+1,-1}, in the model's storage precision.
__device__ __forceinline__ float perturb_f32(float w, float signed_eps) { return w + signed_eps; }
__device__ __forceinline__ uint32_t perturb_bf16(uint32_t w16, float signed_eps) {
  return f32_to_bf16_rne(bf16_to_f32(w16) + signed_eps);
}

// Signed epsilon from a sign bit: bit set -> -eps.
__device__ __forceinline__ float signed_eps(float eps, uint32_t bit) {
  return __uint_as_float(__float_as_uint(eps) ^ (bit << 31));
}

__global__ void k_seeds(uint64_t base_seed, uint64_t step, int n, uint64_t* seeds) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) seeds[i] = probe_seed(base_seed, step, static_cast<uint32_t>(i));
}

// Checks one step's inputs and targets and counts the positions that are scored. Input (b, t)
// is in[b * in_stride + t], target (b, t) is tg[b * tg_stride + t]; a target below zero marks a
// position that is not scored, which only the transduction form allows (allow_unscored).
// flags[1] = 1 if an input lies outside [0, V), a target at or above V, or (when unscored targets
// are not allowed) below zero; else 0. flags[2] = number of scored positions. One block.
__global__ void k_check_tokens(const int32_t* __restrict__ in, int in_stride, const int32_t* __restrict__ tg,
                               int tg_stride, int B, int T, int V, int allow_unscored, uint32_t* flags) {
  __shared__ int bad;
  __shared__ unsigned int scored;
  if (threadIdx.x == 0) {
    bad = 0;
    scored = 0u;
  }
  __syncthreads();
  int mine = 0;
  unsigned int count = 0u;
  const int64_t n = static_cast<int64_t>(B) * T;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t b = i / T, t = i - b * T;
    const int x = in[b * in_stride + t];
    const int y = tg[b * tg_stride + t];
    mine |= (x < 0 || x >= V || y >= V || (y < 0 && !allow_unscored)) ? 1 : 0;
    count += (y >= 0) ? 1u : 0u;
  }
  if (mine) atomicOr(&bad, 1);
  atomicAdd(&scored, count);
  __syncthreads();
  if (threadIdx.x == 0) {
    flags[1] = static_cast<uint32_t>(bad);
    flags[2] = scored;
  }
}

// The two probe-independent candidates of every bf16 weight: wp = bf16(w + eps), wm = bf16(w - eps).
// A probe then only selects one of them per element (sign bit), so the perturbed operand is
// formed by a bit select in registers. 8 elements per thread; n may be ragged.
__global__ void k_pm_table_bf16(const uint16_t* __restrict__ w, int64_t n, float eps,
                                uint16_t* __restrict__ wp, uint16_t* __restrict__ wm) {
  const int64_t base = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
  if (base >= n) return;
  if (base + 8 <= n && ((reinterpret_cast<uintptr_t>(w + base) & 15u) == 0)) {
    const uint4 v = *reinterpret_cast<const uint4*>(w + base);
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t p[4], m[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = in[k] & 0xffffu, hi = in[k] >> 16;
      p[k] = perturb_bf16(lo, eps) | (perturb_bf16(hi, eps) << 16);
      m[k] = perturb_bf16(lo, -eps) | (perturb_bf16(hi, -eps) << 16);
    }
    *reinterpret_cast<uint4*>(wp + base) = make_uint4(p[0], p[1], p[2], p[3]);
    *reinterpret_cast<uint4*>(wm + base) = make_uint4(m[0], m[1], m[2], m[3]);
  } else {
    for (int64_t j = base; j < n && j < base + 8; ++j) {
      wp[j] = static_cast<uint16_t>(perturb_bf16(w[j], eps));
      wm[j] = static_cast<uint16_t>(perturb_bf16(w[j], -eps));
    }
  }
}

// The probe sign bits of one recurrent weight tensor [rows][cols] (cols a multiple of 32) for
// the probe pairs pair0 .. pair0 + pc - 1 of a chunk, as 32-bit words stored chunk-major:
// out[q][w][r] covers columns 32w .. 32w + 31 of row r and is word (w & 3) of the Philox block
// w >> 2, so bit ((c & 31) >> 1) | ((c & 1) << 4) of word c >> 5 is the sign bit of column c.
// The gate kernels read the words of one 32-column chunk for runs of consecutive rows (whole
// cache lines) instead of regenerating the same Philox blocks for every timestep and column
// tile. One thread per (pair, 128-column block, row), rows fastest so that stores coalesce.
__global__ void k_sign_words(const uint64_t* __restrict__ seeds, int pair0, int pc, uint32_t tensor,
                             int rows, int wpr, uint32_t* __restrict__ out) {
  const int nblk = (wpr + 3) / 4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(pc) * rows * nblk) return;
  const int r = static_cast<int>(i % rows);
  const int64_t qb = i / rows;
  const int blk = static_cast<int>(qb % nblk);
  const int q = static_cast<int>(qb / nblk);
  const PhiloxOut o = sign_block(seeds[pair0 + q], tensor, static_cast<uint32_t>(r), static_cast<uint32_t>(blk));
  const uint32_t w[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int wi = 4 * blk + k;
    if (wi < wpr) out[(static_cast<int64_t>(q) * wpr + wi) * rows + r] = w[k];
  }
}

// Per-model perturbed copy of a small tensor [rows][cols] of a bf16 model, for models
// m = 0..2P-1 of a chunk (model 2q is probe pair0+q at +eps, 2q+1 the same probe at -eps).
// out_bf16 (if not null) gets bf16 bits at [m][r][out_cols]; out_f32 (if not null) gets the same
// values as floats, or, when `round` is 0, the perturbed value w +- eps itself in float (the
// exact-perturbation model's biases). One thread per (m, r, 32-column group).
__global__ void k_model_tensor_bf16(const uint16_t* __restrict__ src, int rows, int cols,
                                    uint32_t tensor, const uint64_t* __restrict__ seeds, int pair0,
                                    int n_models, float eps, int out_cols, int round,
                                    uint16_t* __restrict__ out_bf16, float* __restrict__ out_f32) {
  const int groups = (cols + 31) / 32;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(n_models) * rows * groups) return;
  const int g = static_cast<int>(idx % groups);
  const int r = static_cast<int>((idx / groups) % rows);
  const int m = static_cast<int>(idx / (static_cast<int64_t>(groups) * rows));
  const uint64_t seed = seeds[pair0 + (m >> 1)];
  const float e = (m & 1) ? -eps : eps;
  const PhiloxOut o = sign_block(seed, tensor, static_cast<uint32_t>(r), static_cast<uint32_t>(g >> 2));
  const uint32_t word = pick_word(o, static_cast<uint32_t>(g & 3));
  for (int j = 0; j < 32; ++j) {
    const int c = g * 32 + j;
    if (c >= cols) break;
    const uint32_t bit = (word >> sign_bit_pos(static_cast<uint32_t>(c))) & 1u;
    const uint32_t w16 = src[static_cast<int64_t>(r) * cols + c];
    const float se = signed_eps(e, bit);
    const uint32_t v = perturb_bf16(w16, se);
    const int64_t o_idx = (static_cast<int64_t>(m) * rows + r) * out_cols + c;
    if (out_bf16) out_bf16[o_idx] = static_cast<uint16_t>(v);
    if (out_f32) out_f32[o_idx] = round ? bf16_to_f32(v) : bf16_to_f32(w16) + se;
  }
}

// Layer-0 input of timestep t for every (model, sequence) column of a chunk: column m * B + b
// holds emb_m[m][token(b, t)][:], the model's perturbed embedding row, stored k-chunk-major
// like the h of a lower layer (element (column, e) at ((e / 32) ncols_pad + column) 32 + e % 32);
// the token of sequence b at t is in[b * in_stride + t]. Columns ncols .. ncols_pad - 1 are zero.
// Tokens outside [0, V) are clamped (the step's losses are NaN then anyway). E % 32 == 0. A thread owns one 16-byte piece of one column in each of
// kGatherChunks consecutive 32-wide chunks (one token lookup for all of them, and their loads in
// flight together); grid (ceil(4 ncols_pad / 256), ceil(E / 32 / kGatherChunks)), and consecutive
// threads write consecutive pieces of a chunk.
constexpr int kGatherChunks = 4;
__global__ void k_gather_x0(const uint16_t* __restrict__ emb_m, const int32_t* __restrict__ in, int in_stride,
                            int B, int t, int V, int E, int ncols, int ncols_pad, uint16_t* __restrict__ x) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;  // 4 column + piece, < 4 ncols_pad
  if (i >= 4u * static_cast<uint32_t>(ncols_pad)) return;
  const uint32_t col = i >> 2, p4 = i & 3, kc0 = blockIdx.y * kGatherChunks;
  const uint32_t nkc = static_cast<uint32_t>(E) / 32u;
  uint4 v[kGatherChunks];
  const uint4* row = nullptr;
  if (col < static_cast<uint32_t>(ncols)) {
    const uint32_t m = col / static_cast<uint32_t>(B), b = col - m * static_cast<uint32_t>(B);
    int tok = in[static_cast<int64_t>(b) * in_stride + t];
    tok = min(max(tok, 0), V - 1);
    row = reinterpret_cast<const uint4*>(emb_m + (static_cast<int64_t>(m) * V + tok) * E);
  }
#pragma unroll
  for (int j = 0; j < kGatherChunks; ++j) {
    const uint32_t kc = kc0 + j;
    v[j] = (row != nullptr && kc < nkc) ? row[4 * kc + p4] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kGatherChunks; ++j) {
    const uint32_t kc = kc0 + j;
    if (kc < nkc) reinterpret_cast<uint4*>(x)[static_cast<int64_t>(kc) * 4 * ncols_pad + i] = v[j];
  }
}

// losses[m0 + m] = (sum_b seq[m][b]) / (number of scored positions, flags[2]; B T for a language
// model) with a fixed-order double reduction (bitwise repeatable); seq_out[m0 + m][b] = seq[m][b]
// when requested. NaN when tokens were invalid or no position is scored.
__global__ void k_loss_reduce(const float* __restrict__ seq, int B, int m0,
                              const uint32_t* __restrict__ flags, float* __restrict__ losses,
                              float* __restrict__ seq_out) {
  __shared__ double part[256];
  const int m = blockIdx.x;
  double s = 0.0;
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const float v = seq[static_cast<int64_t>(m) * B + b];
    s += static_cast<double>(v);
    if (seq_out) seq_out[static_cast<int64_t>(m0 + m) * B + b] = v;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float mean = static_cast<float>(part[0] / static_cast<double>(flags[2]));
    losses[m0 + m] = (flags[1] || flags[2] == 0u) ? __builtin_nanf("") : mean;
  }
}

// ---------------------------------------------------------------------------------------------
// Seed-regenerating update: theta_j <- theta_j - coef * sum_i d_i p_i(j), d_i = L+_i - L-_i.
// One launch per tensor [rows][cols]. A block covers 16 row segments of 128 columns; 16 threads
// share a segment, each owning 8 consecutive columns (coalesced 16/32-byte accesses). The 128-bit
// Philox words of (probe, segment) are computed once by one of the 16 threads and shared
// through LDS. Non-finite losses: nothing is written and flags[0] is raised.
// ---------------------------------------------------------------------------------------------
constexpr int kUpdThreads = 256;
constexpr int kUpdProbeGroup = 64;

template <bool BF16>
__global__ __launch_bounds__(kUpdThreads) void k_update(
    void* __restrict__ theta_tensor, int rows, int cols, uint32_t tensor,
    const uint64_t* __restrict__ seeds, const float* __restrict__ losses, int K, float coef,
    uint32_t* __restrict__ flags) {
  __shared__ float dif[1024];
  __shared__ uint64_t sseed[kUpdProbeGroup];
  __shared__ uint32_t words[16][kUpdProbeGroup][5];
  __shared__ int bad;
  const int tid = threadIdx.x;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int i = tid; i < K; i += kUpdThreads) {
    const float lp = losses[2 * i], lm = losses[2 * i + 1];
    if (!isfinite(lp) || !isfinite(lm)) atomicOr(&bad, 1);
    dif[i] = lp - lm;
  }
  __syncthreads();
  if (bad) {
    if (tid == 0 && blockIdx.x == 0) flags[0] = 1u;
    return;
  }
  const int segs_per_row = (cols + 127) / 128;
  const int64_t seg = static_cast<int64_t>(blockIdx.x) * 16 + (tid >> 4);
  const int q = tid & 15;
  const bool seg_ok = seg < static_cast<int64_t>(rows) * segs_per_row;
  const int r = seg_ok ? static_cast<int>(seg / segs_per_row) : 0;
  const int blk = seg_ok ? static_cast<int>(seg % segs_per_row) : 0;
  const int c0 = blk * 128 + 8 * q;

  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;

  for (int g0 = 0; g0 < K; g0 += kUpdProbeGroup) {
    const int ng = min(kUpdProbeGroup, K - g0);
    __syncthreads();
    for (int i = tid; i < ng; i += kUpdThreads) sseed[i] = seeds[g0 + i];
    __syncthreads();
    if (seg_ok) {
      for (int i = q; i < ng; i += 16) {
        const PhiloxOut o = sign_block(sseed[i], tensor, static_cast<uint32_t>(r), static_cast<uint32_t>(blk));
        words[tid >> 4][i][0] = o.x;
        words[tid >> 4][i][1] = o.y;
        words[tid >> 4][i][2] = o.z;
        words[tid >> 4][i][3] = o.w;
      }
    }
    __syncthreads();
    if (seg_ok) {
      // Columns c0..c0+7 sit in word (q >> 2); even columns read bits 4(q&3)+0..3, odd columns
      // bits 16+4(q&3)+0..3.
      const int sh = 4 * (q & 3);
      for (int i = 0; i < ng; ++i) {
        const uint32_t w = words[tid >> 4][i][q >> 2];
        const float d = dif[g0 + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t bit = (w >> (sh + (u >> 1) + 16 * (u & 1))) & 1u;
          acc[u] += __uint_as_float(__float_as_uint(d) ^ (bit << 31));
        }
      }
    }
  }
  if (!seg_ok) return;
  const int64_t off = static_cast<int64_t>(r) * cols + c0;
  if (BF16) {
    uint16_t* t = static_cast<uint16_t*>(theta_tensor) + off;
    if (c0 + 8 <= cols && ((reinterpret_cast<uintptr_t>(t) & 15u) == 0)) {
      uint4 v = *reinterpret_cast<const uint4*>(t);
      uint32_t in[4] = {v.x, v.y, v.z, v.w}, out[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = bf16_to_f32(in[k] & 0xffffu) - coef * acc[2 * k];
        const float hi = bf16_to_f32(in[k] >> 16) - coef * acc[2 * k + 1];
        out[k] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
      }
      *reinterpret_cast<uint4*>(t) = make_uint4(out[0], out[1], out[2], out[3]);
    } else {
      for (int u = 0; u < 8 && c0 + u < cols; ++u)
        t[u] = static_cast<uint16_t>(f32_to_bf16_rne(bf16_to_f32(t[u]) - coef * acc[u]));
    }
  } else {
    float* t = static_cast<float*>(theta_tensor) + off;
    if (c0 + 8 <= cols && ((reinterpret_cast<uintptr_t>(t) & 15u) == 0)) {
      float4 a = reinterpret_cast<const float4*>(t)[0];
      float4 b = reinterpret_cast<const float4*>(t)[1];
      a.x -= coef * acc[0]; a.y -= coef * acc[1]; a.z -= coef * acc[2]; a.w -= coef * acc[3];
      b.x -= coef * acc[4]; b.y -= coef * acc[5]; b.z -= coef * acc[6]; b.w -= coef * acc[7];
      reinterpret_cast<float4*>(t)[0] = a;
      reinterpret_cast<float4*>(t)[1] = b;
    } else {
      for (int u = 0; u < 8 && c0 + u < cols; ++u) t[u] -= coef * acc[u];
    }
  }
}

// LSTM cell from the four gate pre-activations: sigmoid(x) = 1 / (1 + e^-x),
// tanh(x) = 2 / (1 + e^-2x) - 1, c' = sigmoid(f) c + sigmoid(i) tanh(g), h = sigmoid(o) tanh(c').
// Written this way the functions saturate correctly without clamping (e^-x = inf gives 0 and
// -1) and a NaN argument stays NaN; each cell costs 5 exponentials and 5 reciprocals.
__device__ __forceinline__ float cell_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float cell_tanh(float x) {
  return 2.f * __builtin_amdgcn_rcpf(1.f + __expf(-2.f * x)) - 1.f;
}
__device__ __forceinline__ void lstm_cell(float gi, float gf, float gg, float go, float c, float& c_out,
                                          float& h_out) {
  const float cn = cell_sigmoid(gf) * c + cell_sigmoid(gi) * cell_tanh(gg);
  c_out = cn;
  h_out = cell_sigmoid(go) * cell_tanh(cn);
}

}  // namespace cdrge
