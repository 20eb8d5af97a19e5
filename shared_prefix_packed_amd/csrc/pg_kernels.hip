// Position ids, rotary embedding and the plain per-row attention kernel.
//
// Position ids follow the verl prefix_grouper_utils.py page (section 1,
// building position ids): prefix tokens count from 0, every suffix restarts at
// the prefix length. RoPE is applied at those positions (the pages never define
// RoPE; rotate-half convention). The per-row attention kernel evaluates the
// packed key set of every token directly (fp32, and bf16 with d = 64).
#include <hip/hip_runtime.h>

#include "pg_hip_common.h"
#include "pg_internal.h"

namespace {

using pg_hip::rope_hi;
using pg_hip::rope_lo;

// ------------------------------------------------------------- positions --
// One thread per token: pos = t - g0 in the prefix, P + (t - ss) in a suffix.
__global__ __launch_bounds__(256) void positions_kernel(const int32_t* __restrict__ g0,
                                                        const int32_t* __restrict__ pe,
                                                        const int32_t* __restrict__ ss,
                                                        int64_t* __restrict__ pos, int32_t T) {
  const int32_t t = int32_t(blockIdx.x) * 256 + int32_t(threadIdx.x);
  if (t >= T) return;
  const int32_t a = g0[t], p = pe[t];
  pos[t] = t < p ? int64_t(t - a) : int64_t(p - a) + int64_t(t - ss[t]);
}

// ------------------------------------------------------------------ RoPE --
// A workgroup handles ROPE_TOK tokens. First every (token, i) angle's cos/sin
// is taken in fp64 and parked in LDS; then each thread rotates chunks of 8
// pairs (x_i.., x_{i+d/2}..) of one head with 16-byte loads for bf16. The
// rotation runs in fp64 and is rounded once to the storage dtype: in fp32,
// x cos - y sin loses to cancellation near zero more than a bf16 ulp there.
constexpr int ROPE_TOK = 2;

template <typename T>
struct Vec8;
template <>
struct Vec8<uint16_t> {   // 8 bf16 as raw bits
  // Q and K stream through once: non-temporal loads and stores keep them
  // from displacing other lines in the caches (4-10 % faster on the
  // larger workloads)
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  uint4 v;
  __device__ void load(const uint16_t* p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    v = make_uint4(t.x, t.y, t.z, t.w);
  }
  __device__ void store(uint16_t* p) const {
    const u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
  }
  __device__ double get(int e) const {
    const uint32_t w = (&v.x)[e >> 1];
    return double(__uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16)));
  }
  // Each value is rounded to fp32 by rounding to odd (truncate, and set the
  // last bit when anything was cut off), then to bf16 by nearest-even in one
  // v_cvt_pk_bf16_f32: with 16 bits to spare the two roundings give the
  // nearest-even bf16 of the fp64 value (Boldo and Melquiond's rounding to
  // odd), without 64-bit integer arithmetic.
  __device__ static float to_f32_odd(double d) {
    const float r = float(d);   // nearest-even
    const double back = double(r);
    uint32_t b = __float_as_uint(r);
    if (back != d) {
      if (__builtin_fabs(back) > __builtin_fabs(d)) b -= 1u;   // rounded away: truncate
      b |= 1u;
    }
    return __uint_as_float(b);
  }
  __device__ void set2(int m, double a, double b) {
    (&v.x)[m] = pg_hip::pack_bf16x2(to_f32_odd(a), to_f32_odd(b));
  }
};
template <>
struct Vec8<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ void store(float* p) const {
    *reinterpret_cast<float4*>(p) = a;
    *reinterpret_cast<float4*>(p + 4) = b;
  }
  __device__ double get(int e) const { return double(e < 4 ? (&a.x)[e] : (&b.x)[e - 4]); }
  __device__ void set2(int m, double x, double y) {
    float* f = m < 2 ? &a.x : &b.x;
    f[(2 * m) & 3] = float(x);
    f[(2 * m + 1) & 3] = float(y);
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kernel(const int64_t* __restrict__ pos,
                                                   const double* __restrict__ inv_freq,
                                                   const T* q_in, const T* k_in, T* q_out,
                                                   T* k_out, int32_t Ttok, int32_t Hq,
                                                   int32_t Hkv) {
  constexpr int HALF = D / 2;
  constexpr int NCH = HALF / 8;
  __shared__ double cs[ROPE_TOK][HALF];
  __shared__ double sn[ROPE_TOK][HALF];
  const int64_t tbase = int64_t(blockIdx.x) * ROPE_TOK;
  for (int e = threadIdx.x; e < ROPE_TOK * HALF; e += 256) {
    const int tt = e / HALF, i = e % HALF;
    const int64_t t = tbase + tt;
    double s = 0.0, c = 1.0;
    if (t < Ttok) sincos(double(pos[t]) * inv_freq[i], &s, &c);
    cs[tt][i] = c;
    sn[tt][i] = s;
  }
  __syncthreads();
  const int heads = Hq + Hkv;
  const int tasks = ROPE_TOK * heads * NCH;
  for (int task = threadIdx.x; task < tasks; task += 256) {
    const int tt = task / (heads * NCH);
    const int rem = task - tt * heads * NCH;
    const int hh = rem / NCH;
    const int ch = rem - hh * NCH;
    const int64_t t = tbase + tt;
    if (t >= Ttok) continue;
    const T* src;
    T* dst;
    if (hh < Hq) {
      if (!q_in) continue;   // K only
      src = q_in + (t * Hq + hh) * D;
      dst = q_out + (t * Hq + hh) * D;
    } else {
      if (!k_in) continue;   // Q only
      src = k_in + (t * Hkv + (hh - Hq)) * D;
      dst = k_out + (t * Hkv + (hh - Hq)) * D;
    }
    Vec8<T> lo, hi, ylo, yhi;
    lo.load(src + ch * 8);
    hi.load(src + HALF + ch * 8);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      double rl[2], rh[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int e = 2 * m + e2;
        const double c = cs[tt][ch * 8 + e], s = sn[tt][ch * 8 + e];
        const double xl = lo.get(e), xh = hi.get(e);
        rl[e2] = rope_lo(xl, xh, c, s);
        rh[e2] = rope_hi(xl, xh, c, s);
      }
      ylo.set2(m, rl[0], rl[1]);
      yhi.set2(m, rh[0], rh[1]);
    }
    ylo.store(dst + ch * 8);
    yhi.store(dst + HALF + ch * 8);
  }
}

// ------------------------------------------------------ per-row attention --
// One wave per (token, query head). Lanes split the head dimension; the wave
// walks the token's key set K(t) = [g0, pe) u [ss, t] (prefix tokens: [g0, t])
// with an online softmax in base 2. Reference-grade speed, used for fp32 and
// for bf16 with d = 64.
template <typename T>
__device__ inline float to_f(T x);
template <>
__device__ inline float to_f<float>(float x) { return x; }
template <>
__device__ inline float to_f<uint16_t>(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
template <typename T>
__device__ inline T from_f(float x);
template <>
__device__ inline float from_f<float>(float x) { return x; }
template <>
__device__ inline uint16_t from_f<uint16_t>(float x) {
  const uint32_t u = __float_as_uint(x);
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void attn_rowwise_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ o,
    float* __restrict__ lse, const int32_t* __restrict__ g0a, const int32_t* __restrict__ pea,
    const int32_t* __restrict__ ssa, int32_t Ttok, int32_t Hq, int32_t Hkv, float c_log2) {
  constexpr int E = D / 64;
  const int64_t idx = blockIdx.x;
  const int32_t t = int32_t(idx / Hq);
  const int32_t h = int32_t(idx % Hq);
  const int32_t hk = h / (Hq / Hkv);
  const int lane = threadIdx.x;
  float qv[E], acc[E];
  const T* qr = q + (int64_t(t) * Hq + h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = to_f<T>(qr[lane * E + e]);
    acc[e] = 0.f;
  }
  const int32_t g0 = g0a[t], pe = pea[t], ss = ssa[t];
  float m = -1.0e30f, l = 0.f;
  for (int32_t j = g0; j <= t; ++j) {
    if (j >= pe && j < ss) j = ss;   // skip sibling suffixes (ss <= t always)
    const T* kr = k + (int64_t(j) * Hkv + hk) * D;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) part += qv[e] * to_f<T>(kr[lane * E + e]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    const float s = part * c_log2;
    const float mn = fmaxf(m, s);
    const float alpha = exp2f(m - mn);
    const float p = exp2f(s - mn);
    l = l * alpha + p;
    const T* vr = v + (int64_t(j) * Hkv + hk) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = acc[e] * alpha + p * to_f<T>(vr[lane * E + e]);
    m = mn;
  }
  const float inv = 1.f / l;
  T* orow = o + (int64_t(t) * Hq + h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) orow[lane * E + e] = from_f<T>(acc[e] * inv);
  if (lse && lane == 0) lse[int64_t(h) * Ttok + t] = (m + log2f(l)) * 0.69314718055994530942f;
}


// ------------------------------------------------- per-row backward --
// The backward of the per-row forward, for fp32 and for d = 64 (the MFMA
// kernels take bf16 with d = 128): the chain rule as the MFMA path computes
// it, in fp32 from the stored inputs, one wave per row and no matrix units.
// With P the softmax of query row t over K(t) (p_j = exp(scale q.k_j - lse_t),
// from the forward's lse) and D_t = dO_t . O_t (the forward's O as stored):
//   dQ_t = scale sum_j p_j (dO_t . v_j - D_t) k_j            (query rows)
//   dV_j = sum p_tj dO_t,  dK_j = scale sum p_tj (dO_t . v_j - D_t) q_t
// over the query rows t that read key j and the query heads of its KV head
// (key rows). The rows that read key j are one contiguous range [j, qend):
// the rest of the group for a prompt key (every response reads the whole
// prompt), the rest of its own response otherwise.
// The query-row launch writes D to `delta`; the key-row launch reads it.
template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_rowwise_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ o, const float* __restrict__ lse, const T* __restrict__ dout,
    T* __restrict__ dq, float* __restrict__ delta, const int32_t* __restrict__ g0a,
    const int32_t* __restrict__ pea, const int32_t* __restrict__ ssa, int32_t Ttok, int32_t Hq,
    int32_t Hkv, float c_log2, float scale) {
  constexpr int E = D / 64;
  const int64_t idx = blockIdx.x;
  const int32_t t = int32_t(idx / Hq);
  const int32_t h = int32_t(idx % Hq);
  const int32_t hk = h / (Hq / Hkv);
  const int lane = threadIdx.x;
  const int64_t row = (int64_t(t) * Hq + h) * D;
  float qv[E], gv[E], acc[E];
  float dd = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = to_f<T>(q[row + lane * E + e]);
    gv[e] = to_f<T>(dout[row + lane * E + e]);
    dd += gv[e] * to_f<T>(o[row + lane * E + e]);
    acc[e] = 0.f;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dd += __shfl_xor(dd, off, 64);
  const float l2 = lse[int64_t(h) * Ttok + t] * 1.44269504088896340736f;
  const int32_t g0 = g0a[t], pe = pea[t], ss = ssa[t];
  for (int32_t j = g0; j <= t; ++j) {
    if (j >= pe && j < ss) j = ss;   // skip sibling suffixes (ss <= t always)
    const int64_t kv = (int64_t(j) * Hkv + hk) * D;
    float sp = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      sp += qv[e] * to_f<T>(k[kv + lane * E + e]);
      dp += gv[e] * to_f<T>(v[kv + lane * E + e]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      sp += __shfl_xor(sp, off, 64);
      dp += __shfl_xor(dp, off, 64);
    }
    const float ds = exp2f(sp * c_log2 - l2) * (dp - dd);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += ds * to_f<T>(k[kv + lane * E + e]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) dq[row + lane * E + e] = from_f<T>(acc[e] * scale);
  if (lane == 0) delta[int64_t(h) * Ttok + t] = dd;
}

template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_rowwise_dkv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ delta, const T* __restrict__ dout,
    T* __restrict__ dk, T* __restrict__ dv, const int32_t* __restrict__ pea,
    const int32_t* __restrict__ ssa, const int32_t* __restrict__ owner,
    const int32_t* __restrict__ group_off, const int32_t* __restrict__ suffix_lens,
    int32_t Ttok, int32_t Hq, int32_t Hkv, float c_log2, float scale) {
  constexpr int E = D / 64;
  const int64_t idx = blockIdx.x;
  const int32_t j = int32_t(idx / Hkv);
  const int32_t hk = int32_t(idx % Hkv);
  const int32_t r = Hq / Hkv;
  const int lane = threadIdx.x;
  const int64_t kv = (int64_t(j) * Hkv + hk) * D;
  float kvk[E], kvv[E], ak[E], av[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kvk[e] = to_f<T>(k[kv + lane * E + e]);
    kvv[e] = to_f<T>(v[kv + lane * E + e]);
    ak[e] = 0.f;
    av[e] = 0.f;
  }
  // owner: the group of a prompt token, the response of a response token
  const int32_t qend =
      j < pea[j] ? group_off[owner[j] + 1] : ssa[j] + suffix_lens[owner[j]];
  for (int32_t t = j; t < qend; ++t) {
    for (int32_t h = hk * r; h < hk * r + r; ++h) {
      const int64_t row = (int64_t(t) * Hq + h) * D;
      float qv[E], gv[E];
      float sp = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        qv[e] = to_f<T>(q[row + lane * E + e]);
        gv[e] = to_f<T>(dout[row + lane * E + e]);
        sp += qv[e] * kvk[e];
        dp += gv[e] * kvv[e];
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        sp += __shfl_xor(sp, off, 64);
        dp += __shfl_xor(dp, off, 64);
      }
      const int64_t hr = int64_t(h) * Ttok + t;
      const float p = exp2f(sp * c_log2 - lse[hr] * 1.44269504088896340736f);
      const float ds = p * (dp - delta[hr]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        av[e] += p * gv[e];
        ak[e] += ds * qv[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dk[kv + lane * E + e] = from_f<T>(ak[e] * scale);
    dv[kv + lane * E + e] = from_f<T>(av[e]);
  }
}

// Decode step, one workgroup (one wave) per (response k, query head h): the
// newest token of response k against its group's prompt rows and its first
// len_k = clamp(cur_lens[k], 0, capacity_k) own rows (PackInfer abstract,
// group-contiguous KV cache). Online softmax as in attn_rowwise_kernel. No
// tables (a layout without tokens): every key set is empty.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_rowwise_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ cur_lens, const int32_t* __restrict__ group_off,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ suffix_group, const int32_t* __restrict__ caps,
    T* __restrict__ o, float* __restrict__ lse, int32_t N, int32_t Hq, int32_t Hkv,
    float c_log2) {
  constexpr int E = D / 64;
  const int32_t kr = int32_t(blockIdx.x / Hq);
  const int32_t h = int32_t(blockIdx.x % Hq);
  const int32_t hk = h / (Hq / Hkv);
  const int lane = threadIdx.x;
  float qv[E], acc[E];
  const T* qr = q + (int64_t(kr) * Hq + h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = to_f<T>(qr[lane * E + e]);
    acc[e] = 0.f;
  }
  int32_t a = 0, pe = 0, s0 = 0, s1 = 0;
  if (group_off) {
    const int32_t g = suffix_group[kr];
    a = group_off[g];
    pe = a + prefix_lens[g];
    s0 = seg_off[g + kr + 1];
    s1 = s0 + min(max(cur_lens[kr], 0), caps[kr]);
  }
  float m = -INFINITY, l = 0.f;
  for (int32_t j = a; j < s1; ++j) {
    if (j == pe) j = s0;   // the responses between the prompt and this one
    if (j >= s1) break;
    const T* kp = k + (int64_t(j) * Hkv + hk) * D;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) part += qv[e] * to_f<T>(kp[lane * E + e]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    const float s = part * c_log2;
    const float mn = fmaxf(m, s);
    const float alpha = exp2f(m - mn);
    const float p = exp2f(s - mn);
    l = l * alpha + p;
    const T* vp = v + (int64_t(j) * Hkv + hk) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = acc[e] * alpha + p * to_f<T>(vp[lane * E + e]);
    m = mn;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  T* orow = o + (int64_t(kr) * Hq + h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) orow[lane * E + e] = from_f<T>(acc[e] * inv);
  if (lane == 0)
    lse[int64_t(h) * N + kr] = l > 0.f ? (m + log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

// ------------------------------------------------------- pack and unpack --
// Row gathers either side of the packed path (verl prefix_grouper_utils.py
// page, sections 2-3: concatenating each prompt once with its responses, and
// splitting the output back with the last prompt position included in each
// response part). A row is `upr` units of U (16 bytes when the row size
// allows, else 4). One wave per row (grid-stride over rows): the row's source
// is resolved once from the token tables, then consecutive lanes move
// consecutive units, GATHER_UNROLL loads in flight per lane before the stores.
constexpr int GATHER_UNROLL = 4;

// Every gathered row is written once and read by a later kernel, not by this
// one. When a launch writes more than the last-level cache holds, non-temporal
// stores (nt) keep its output from evicting the rows still to be read (2-20 %
// faster on the larger workloads); a smaller output is stored normally, so the
// next kernel still finds it in the cache. Loads stay ordinary either way.
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void put(uint4* p, uint4 v, bool nt) {
  if (nt) {
    const nt_u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<nt_u32x4*>(p));
  } else {
    *p = v;
  }
}
__device__ __forceinline__ void put(uint32_t* p, uint32_t v, bool nt) {
  if (nt) __builtin_nontemporal_store(v, p); else *p = v;
}

template <typename U>
__device__ __forceinline__ void copy_row(const U* __restrict__ src, U* __restrict__ dst,
                                         int64_t upr, int lane, bool nt) {
  int64_t c = lane;
  for (; c + 64 * (GATHER_UNROLL - 1) < upr; c += 64 * GATHER_UNROLL) {
    U v[GATHER_UNROLL];
#pragma unroll
    for (int i = 0; i < GATHER_UNROLL; ++i) v[i] = src[c + 64 * i];
#pragma unroll
    for (int i = 0; i < GATHER_UNROLL; ++i) put(dst + c + 64 * i, v[i], nt);
  }
  for (; c < upr; c += 64) put(dst + c, src[c], nt);
}

template <typename U>
__device__ __forceinline__ void zero_row(U* __restrict__ dst, int64_t upr, int lane, bool nt) {
  U z;
  __builtin_memset(&z, 0, sizeof(U));
  for (int64_t c = lane; c < upr; c += 64) put(dst + c, z, nt);
}

// packed[t] = prompt row (owner g, index t - g0) or response row (owner k,
// index t - ss).
template <typename U>
__global__ __launch_bounds__(256) void pack_rows_kernel(const int32_t* __restrict__ owner,
                                                        const int32_t* __restrict__ g0,
                                                        const int32_t* __restrict__ pe,
                                                        const int32_t* __restrict__ ss,
                                                        const U* prefix, int64_t ppad,
                                                        const U* suffix, int64_t spad, U* packed,
                                                        int64_t rows, int64_t upr, bool nt) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = int64_t(gridDim.x) * (blockDim.x >> 6);
  for (int64_t t = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6); t < rows;
       t += nw) {
    const int64_t o = owner[t];
    const U* src = t < pe[t] ? prefix + (o * ppad + (t - g0[t])) * upr
                             : suffix + (o * spad + (t - ss[t])) * upr;
    copy_row(src, packed + t * upr, upr, lane, nt);
  }
}

// Output rows: prompt part [G, ppad] (row i of group g: packed row
// group_off[g] + i if i < prefix_lens[g]), response part [N, spad + 1] (row 0:
// the group's last prompt row; row 1 + j: response row j); zeros elsewhere and
// everywhere when the layout has no tokens (no tables).
template <typename U>
__global__ __launch_bounds__(256) void unpack_rows_kernel(
    const int32_t* __restrict__ group_off, const int32_t* __restrict__ prefix_lens,
    const int32_t* __restrict__ seg_off, const int32_t* __restrict__ suffix_group,
    const int32_t* __restrict__ suffix_lens, const U* packed, U* prefix_out, int64_t G,
    int64_t ppad, U* suffix_out, int64_t N, int64_t spad, int64_t upr, bool nt) {
  const int64_t pre_rows = prefix_out ? G * ppad : 0;
  const int64_t suf_rows = suffix_out ? N * (spad + 1) : 0;
  const int64_t rows = pre_rows + suf_rows;
  const bool have = group_off != nullptr;
  const int lane = threadIdx.x & 63;
  const int64_t nw = int64_t(gridDim.x) * (blockDim.x >> 6);
  for (int64_t row = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6); row < rows;
       row += nw) {
    int64_t src = -1;
    U* dst;
    if (row < pre_rows) {
      const int64_t g = row / ppad, i = row - g * ppad;
      if (have && i < prefix_lens[g]) src = group_off[g] + i;
      dst = prefix_out + row * upr;
    } else {
      const int64_t r = row - pre_rows;
      const int64_t k = r / (spad + 1), j = r - k * (spad + 1);
      if (have) {
        const int32_t g = suffix_group[k];
        if (j == 0) {
          if (prefix_lens[g] > 0) src = group_off[g] + prefix_lens[g] - 1;
        } else if (j - 1 < suffix_lens[k]) {
          src = seg_off[g + k + 1] + (j - 1);   // response k is segment g + k + 1
        }
      }
      dst = suffix_out + r * upr;
    }
    if (src >= 0)
      copy_row(packed + src * upr, dst, upr, lane, nt);
    else
      zero_row(dst, upr, lane, nt);
  }
}

}  // namespace

hipError_t pg_launch_positions(const pg_layout& L, int64_t* pos, hipStream_t stream) {
  const int32_t T = int32_t(L.T);
  positions_kernel<<<dim3((T + 255) / 256), dim3(256), 0, stream>>>(L.d_g0, L.d_pe, L.d_ss, pos, T);
  return hipGetLastError();
}

hipError_t pg_launch_rope(const pg_layout& L, const int64_t* pos, const void* q_in,
                          const void* k_in, void* q_out, void* k_out, pg_dtype dtype,
                          hipStream_t stream) {
  const int32_t T = int32_t(L.T);
  const dim3 grid((T + ROPE_TOK - 1) / ROPE_TOK), block(256);
#define PG_ROPE(TY, DD)                                                                       \
  rope_kernel<TY, DD><<<grid, block, 0, stream>>>(                                            \
      pos, L.d_inv_freq, static_cast<const TY*>(q_in), static_cast<const TY*>(k_in),          \
      static_cast<TY*>(q_out), static_cast<TY*>(k_out), T, L.Hq, L.Hkv)
  if (dtype == PG_BF16) {
    if (L.d == 128) PG_ROPE(uint16_t, 128); else PG_ROPE(uint16_t, 64);
  } else {
    if (L.d == 128) PG_ROPE(float, 128); else PG_ROPE(float, 64);
  }
#undef PG_ROPE
  return hipGetLastError();
}

hipError_t pg_launch_bwd_rowwise(const pg_layout& L, const void* q, const void* k, const void* v,
                                 const void* o, const float* lse, const void* dout, void* dq,
                                 void* dk, void* dv, float* delta, pg_dtype dtype,
                                 float softmax_scale, hipStream_t stream) {
  const int64_t qrows = L.T * L.Hq, krows = L.T * L.Hkv;
  if (qrows > int64_t(0x7fffffff)) return hipErrorInvalidConfiguration;
  if (qrows == 0) return hipSuccess;
  const float c = softmax_scale * 1.44269504088896340736f;
  const int32_t T = int32_t(L.T);
#define PG_BWD(TY, DD)                                                                          \
  do {                                                                                          \
    bwd_rowwise_dq_kernel<TY, DD><<<dim3(uint32_t(qrows)), dim3(64), 0, stream>>>(              \
        static_cast<const TY*>(q), static_cast<const TY*>(k), static_cast<const TY*>(v),         \
        static_cast<const TY*>(o), lse, static_cast<const TY*>(dout), static_cast<TY*>(dq),      \
        delta, L.d_g0, L.d_pe, L.d_ss, T, L.Hq, L.Hkv, c, softmax_scale);                        \
    bwd_rowwise_dkv_kernel<TY, DD><<<dim3(uint32_t(krows)), dim3(64), 0, stream>>>(             \
        static_cast<const TY*>(q), static_cast<const TY*>(k), static_cast<const TY*>(v), lse,    \
        delta, static_cast<const TY*>(dout), static_cast<TY*>(dk), static_cast<TY*>(dv),         \
        L.d_pe, L.d_ss, L.d_owner, L.d_group_off, L.d_suffix_lens, T, L.Hq, L.Hkv, c,            \
        softmax_scale);                                                                         \
  } while (0)
  if (dtype == PG_BF16) {
    if (L.d == 128) PG_BWD(uint16_t, 128); else PG_BWD(uint16_t, 64);
  } else {
    if (L.d == 128) PG_BWD(float, 128); else PG_BWD(float, 64);
  }
#undef PG_BWD
  return hipGetLastError();
}

hipError_t pg_launch_attn_rowwise(const pg_layout& L, const void* q, const void* k,
                                  const void* v, void* o, float* lse, pg_dtype dtype,
                                  float softmax_scale, hipStream_t stream) {
  const int64_t blocks = L.T * L.Hq;
  if (blocks > int64_t(0x7fffffff)) return hipErrorInvalidConfiguration;
  const float c = softmax_scale * 1.44269504088896340736f;
  const int32_t T = int32_t(L.T);
#define PG_ROW(TY, DD)                                                                        \
  attn_rowwise_kernel<TY, DD><<<dim3(uint32_t(blocks)), dim3(64), 0, stream>>>(             \
      static_cast<const TY*>(q), static_cast<const TY*>(k), static_cast<const TY*>(v),        \
      static_cast<TY*>(o), lse, L.d_g0, L.d_pe, L.d_ss, T, L.Hq, L.Hkv, c)
  if (dtype == PG_BF16) {
    if (L.d == 128) PG_ROW(uint16_t, 128); else PG_ROW(uint16_t, 64);
  } else {
    if (L.d == 128) PG_ROW(float, 128); else PG_ROW(float, 64);
  }
#undef PG_ROW
  return hipGetLastError();
}

hipError_t pg_launch_decode_rowwise(const pg_layout& L, const void* q, const void* k,
                                   const void* v, const int32_t* cur_lens, void* o, float* lse,
                                   pg_dtype dtype, float softmax_scale, hipStream_t stream) {
  const int32_t N = int32_t(L.suffix_lens.size());
  const int64_t blocks = int64_t(N) * L.Hq;
  if (blocks == 0) return hipSuccess;
  const float c = softmax_scale * 1.44269504088896340736f;
  const bool have = L.T > 0 && L.d_group_off != nullptr;
  const int32_t* go = have ? L.d_group_off : nullptr;
#define PG_DEC(TY, DD)                                                                        \
  decode_rowwise_kernel<TY, DD><<<dim3(uint32_t(blocks)), dim3(64), 0, stream>>>(           \
      static_cast<const TY*>(q), static_cast<const TY*>(k), static_cast<const TY*>(v),        \
      cur_lens, go, L.d_prefix_lens, L.d_seg_off, L.d_suffix_group, L.d_suffix_lens,          \
      static_cast<TY*>(o), lse, N, L.Hq, L.Hkv, c)
  if (dtype == PG_BF16) {
    if (L.d == 128) PG_DEC(uint16_t, 128); else PG_DEC(uint16_t, 64);
  } else {
    if (L.d == 128) PG_DEC(float, 128); else PG_DEC(float, 64);
  }
#undef PG_DEC
  return hipGetLastError();
}

namespace {
// ------------------------------------------------------ right-padded form --
// [G, max_len] rows: row g is group g's packed row [group_off[g],
// group_off[g + 1]), then padding (verl page, sections 1-2). No tables (a
// layout without tokens): every group is empty.

// One thread per (g, j): the packed position of token group_off[g] + j, or 0
// on padding; mask 1 on real tokens.
__global__ __launch_bounds__(256) void positions_padded_kernel(
    const int32_t* __restrict__ group_off, const int32_t* __restrict__ g0a,
    const int32_t* __restrict__ pea, const int32_t* __restrict__ ssa, int64_t* __restrict__ pos,
    uint8_t* __restrict__ mask, int64_t G, int32_t max_len) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= G * max_len) return;
  const int64_t g = e / max_len;
  const int32_t j = int32_t(e - g * max_len);
  int64_t p = 0;
  bool real = false;
  if (group_off) {
    const int32_t a = group_off[g];
    if (j < group_off[g + 1] - a) {
      const int32_t t = a + j, pe = pea[t], g0 = g0a[t];
      p = t < pe ? int64_t(t - g0) : int64_t(pe - g0) + int64_t(t - ssa[t]);
      real = true;
    }
  }
  pos[e] = p;
  if (mask) mask[e] = real ? 1 : 0;
}

// One wave per padded row (g, j): the packed row, or zeros on padding.
template <typename U>
__global__ __launch_bounds__(256) void pad_rows_kernel(const int32_t* __restrict__ group_off,
                                                       const U* packed, U* padded, int64_t G,
                                                       int32_t max_len, int64_t upr, bool nt) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = G * max_len;
  const int64_t nw = int64_t(gridDim.x) * (blockDim.x >> 6);
  for (int64_t row = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6); row < rows;
       row += nw) {
    const int64_t g = row / max_len;
    const int32_t j = int32_t(row - g * max_len);
    U* dst = padded + row * upr;
    const int32_t a = group_off ? group_off[g] : 0;
    if (group_off && j < group_off[g + 1] - a)
      copy_row(packed + (int64_t(a) + j) * upr, dst, upr, lane, nt);
    else
      zero_row(dst, upr, lane, nt);
  }
}

// One wave per packed row t: its group (prompt tokens carry it as owner,
// response tokens through their response) and index t - g0 in the group row.
template <typename U>
__global__ __launch_bounds__(256) void unpad_rows_kernel(
    const int32_t* __restrict__ owner, const int32_t* __restrict__ suffix_group,
    const int32_t* __restrict__ g0a, const int32_t* __restrict__ pea, const U* padded, U* packed,
    int64_t T, int32_t max_len, int64_t upr, bool nt) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = int64_t(gridDim.x) * (blockDim.x >> 6);
  for (int64_t t = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6); t < T; t += nw) {
    const int32_t o = owner[t];
    const int64_t g = t < pea[t] ? o : suffix_group[o];
    copy_row(padded + (g * max_len + (t - g0a[t])) * upr, packed + t * upr, upr, lane, nt);
  }
}

// Four rows (waves) per 256-thread block, at most 8192 blocks (32 waves per CU).
dim3 gather_grid(int64_t rows) {
  const int64_t blocks = (rows + 3) / 4;
  return dim3(uint32_t(blocks < 8192 ? (blocks > 0 ? blocks : 1) : 8192));
}

// Streaming stores for launches that write more than MI355X's 256 MB
// last-level cache.
bool stream_out(int64_t rows, int64_t row_bytes) { return rows * row_bytes > (int64_t(256) << 20); }
}  // namespace

hipError_t pg_launch_pack(const pg_layout& L, const void* prefix, int32_t prefix_pad,
                          const void* suffix, int32_t suffix_pad, void* packed, int64_t row_bytes,
                          hipStream_t stream) {
  if (L.T == 0) return hipSuccess;
  if (row_bytes % 16 == 0) {
    const int64_t upr = row_bytes / 16;
    pack_rows_kernel<uint4><<<gather_grid(L.T), dim3(256), 0, stream>>>(
        L.d_owner, L.d_g0, L.d_pe, L.d_ss, static_cast<const uint4*>(prefix), prefix_pad,
        static_cast<const uint4*>(suffix), suffix_pad, static_cast<uint4*>(packed), L.T, upr,
        stream_out(L.T, row_bytes));
  } else {
    const int64_t upr = row_bytes / 4;
    pack_rows_kernel<uint32_t><<<gather_grid(L.T), dim3(256), 0, stream>>>(
        L.d_owner, L.d_g0, L.d_pe, L.d_ss, static_cast<const uint32_t*>(prefix), prefix_pad,
        static_cast<const uint32_t*>(suffix), suffix_pad, static_cast<uint32_t*>(packed), L.T,
        upr, stream_out(L.T, row_bytes));
  }
  return hipGetLastError();
}

hipError_t pg_launch_unpack(const pg_layout& L, const void* packed, int64_t row_bytes,
                            void* prefix_out, int32_t prefix_pad, void* suffix_out,
                            int32_t suffix_pad, hipStream_t stream) {
  const int64_t G = int64_t(L.group_off.size()) - 1, N = int64_t(L.suffix_lens.size());
  const int64_t rows = (prefix_out ? G * prefix_pad : 0) + (suffix_out ? N * (suffix_pad + 1) : 0);
  if (rows == 0) return hipSuccess;
  const bool have = L.T > 0;   // a layout without tokens has no device tables: all zeros
  const int32_t* go = have ? L.d_group_off : nullptr;
  if (row_bytes % 16 == 0)
    unpack_rows_kernel<uint4><<<gather_grid(rows), dim3(256), 0, stream>>>(
        go, L.d_prefix_lens, L.d_seg_off, L.d_suffix_group, L.d_suffix_lens,
        static_cast<const uint4*>(packed), static_cast<uint4*>(prefix_out), G, prefix_pad,
        static_cast<uint4*>(suffix_out), N, suffix_pad, row_bytes / 16, stream_out(rows, row_bytes));
  else
    unpack_rows_kernel<uint32_t><<<gather_grid(rows), dim3(256), 0, stream>>>(
        go, L.d_prefix_lens, L.d_seg_off, L.d_suffix_group, L.d_suffix_lens,
        static_cast<const uint32_t*>(packed), static_cast<uint32_t*>(prefix_out), G, prefix_pad,
        static_cast<uint32_t*>(suffix_out), N, suffix_pad, row_bytes / 4, stream_out(rows, row_bytes));
  return hipGetLastError();
}

hipError_t pg_launch_positions_padded(const pg_layout& L, int32_t max_len, int64_t* pos,
                                      uint8_t* mask, hipStream_t stream) {
  const int64_t G = int64_t(L.group_off.size()) - 1, n = G * max_len;
  if (n == 0) return hipSuccess;
  const bool have = L.T > 0;
  positions_padded_kernel<<<dim3(uint32_t((n + 255) / 256)), dim3(256), 0, stream>>>(
      have ? L.d_group_off : nullptr, L.d_g0, L.d_pe, L.d_ss, pos, mask, G, max_len);
  return hipGetLastError();
}

hipError_t pg_launch_pad(const pg_layout& L, const void* packed, int64_t row_bytes, void* padded,
                         int32_t max_len, hipStream_t stream) {
  const int64_t G = int64_t(L.group_off.size()) - 1, rows = G * max_len;
  if (rows == 0) return hipSuccess;
  const int32_t* go = L.T > 0 ? L.d_group_off : nullptr;
  if (row_bytes % 16 == 0)
    pad_rows_kernel<uint4><<<gather_grid(rows), dim3(256), 0, stream>>>(
        go, static_cast<const uint4*>(packed), static_cast<uint4*>(padded), G, max_len,
        row_bytes / 16, stream_out(rows, row_bytes));
  else
    pad_rows_kernel<uint32_t><<<gather_grid(rows), dim3(256), 0, stream>>>(
        go, static_cast<const uint32_t*>(packed), static_cast<uint32_t*>(padded), G, max_len,
        row_bytes / 4, stream_out(rows, row_bytes));
  return hipGetLastError();
}

hipError_t pg_launch_unpad(const pg_layout& L, const void* padded, int32_t max_len,
                           int64_t row_bytes, void* packed, hipStream_t stream) {
  if (L.T == 0) return hipSuccess;
  if (row_bytes % 16 == 0)
    unpad_rows_kernel<uint4><<<gather_grid(L.T), dim3(256), 0, stream>>>(
        L.d_owner, L.d_suffix_group, L.d_g0, L.d_pe, static_cast<const uint4*>(padded),
        static_cast<uint4*>(packed), L.T, max_len, row_bytes / 16, stream_out(L.T, row_bytes));
  else
    unpad_rows_kernel<uint32_t><<<gather_grid(L.T), dim3(256), 0, stream>>>(
        L.d_owner, L.d_suffix_group, L.d_g0, L.d_pe, static_cast<const uint32_t*>(padded),
        static_cast<uint32_t*>(packed), L.T, max_len, row_bytes / 4, stream_out(L.T, row_bytes));
  return hipGetLastError();
}
