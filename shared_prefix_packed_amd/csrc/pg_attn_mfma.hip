// Packed shared-prefix attention forward, bf16, d = 128, for gfx950 (CDNA4).
//
// What is computed: for every token t and query head h, softmax over the
// packed key set K(t) (own group, j <= t, prefix or own segment) of scaled
// q.k, times V, plus lse = ln(sum exp(scaled scores)). This equals causal
// attention over the unpacked sequence prefix || own suffix ("Preference
// Packing", core idea; verl prefix_grouper_utils.py page, prefix-sharing
// diagram). Tiles are built over the packed query-key region and fully masked
// tiles are never visited ("PackInfer", abstract).
//
// Work item (one workgroup of 4 waves): query tokens [t0, t1) of one group and
// `hpw` query heads of one KV head; wave w takes head hq0 + w % hpw and the
// 32-token block w / hpw. All waves share every K/V tile staged in LDS, so a
// tile fetched once serves hpw heads (GQA) and every suffix in the block (the
// prefix keys are common to all of them).
//
// Per wave and 64-key tile, with 32x32x16 bf16 MFMAs:
//   S^T[key][query] = K . Q^T     A = K rows from LDS, B = Q from registers
//   online softmax per query      one query per lane, keys split over the two
//                                 lane halves: 31 in-lane max/add + 1 swap
//   O^T[d][query]  += V^T . P^T   A = V^T from LDS, B = P straight from the
//                                 S^T accumulators (no transpose needed)
// V is transposed while it is staged into LDS; the key order inside each
// 16-key step is permuted the same way for P and V, so every LDS read is one
// 128-bit access. K rows are padded to 272 bytes and the 16-byte chunks of V^T
// row d are XOR-swizzled by (d >> 1) & 7, which keeps reads and writes free of
// bank conflicts on the 64 four-byte banks of a gfx950 LDS.
#include <hip/hip_runtime.h>

#include "pg_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));


constexpr int D = 128;
constexpr int KT = PG_KEY_TILE;         // 64 keys per tile
constexpr int QW = PG_WAVE_QUERIES;     // 32 queries per wave
constexpr int K_PITCH = 272;            // bytes per K row in LDS (256 + 16 pad)
constexpr int K_BYTES = KT * K_PITCH;   // 17408
constexpr int V_BYTES = D * KT * 2;     // 16384: V^T, 128 bytes per d row
constexpr int STAGE = K_BYTES + V_BYTES;

struct MfmaArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const pg_work_item* items;
  const pg_key_span* spans;
  const int32_t* tok_ss;
  int32_t T, Hq, Hkv, r, hpw;
  float c_log2;   // softmax_scale * log2(e)
};

__device__ inline uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Raw buffer resource over `bytes` bytes from `base` (gfx9 dword3: untyped
// 32-bit data format). A load whose offset lies at or past `bytes` returns
// zeros, so rows past the end of a key span need no clamping.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ inline uint4 buf16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

__device__ inline bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  // nearest-even fp32 -> bf16 of two values in one v_cvt_pk_bf16_f32
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// The running max is raised only when a tile's max exceeds it by more than
// this many powers of two; until then exp2 arguments stay <= 8 and O, l are
// not rescaled. The result is exact either way: numerator and denominator
// share the same stale max.
constexpr float RESCALE_SLACK = 8.0f;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt fields left at "no wait").
// Issued once before the tile loop so every load made before it is known to
// have landed; otherwise the loop's wait counters also cover those loads and
// each tile would wait for the next tile's prefetch as well.
__device__ inline void wait_all_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_d128(MfmaArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const pg_work_item it = a.items[blockIdx.x];
  if (it.nspan == 0) return;   // padding of a shorter XCD queue
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int qi = lane & 31;     // query column of this lane inside the wave
  const int half = lane >> 5;   // which half of each 16-wide k step the lane feeds

  const int h = it.hq0 + wave % a.hpw;
  const int hk = it.hq0 / a.r;   // one KV head per item
  const int tb = it.t0 + QW * (wave / a.hpw);
  const int te = min(tb + QW, it.t1);
  const bool wave_active = tb < te;
  const int tq = wave_active ? min(tb + qi, te - 1) : it.t0;   // padded rows repeat the last one
  const bool row_valid = wave_active && (tb + qi < te);

  // Q as the B operand of S^T = K Q^T: lane holds d = 16 ks + 8 half + 0..7.
  bf16x8_t qf[8];
  {
    const uint16_t* qrow = a.q + (int64_t(tq) * a.Hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(ldg16(qrow + 16 * ks));
  }
  const int ss_t = a.tok_ss[tq];
  int ss_max = ss_t;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss_max = max(ss_max, __shfl_xor(ss_max, off, 64));

  f32x16_t acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m_run = -1.0e30f;   // finite start: exp2(m_run - m_new) is 0, never NaN
  float l_run = 0.f;

  // Staging roles. K: 16 lanes per 256-byte row, rows kr + 16 i.
  // V: lane takes keys 4 va .. 4 va + 3 and d = 8 vc .. 8 vc + 7.
  // Per-lane byte offsets from the tile's first row are fixed; only the
  // scalar base of the buffer resource moves from tile to tile.
  const int kc = tid & 15, kr = tid >> 4;
  const int va = tid & 15, vc = tid >> 4;
  const int row_bytes = a.Hkv * D * 2;
  int koff[4], voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    koff[i] = (kr + 16 * i) * row_bytes + 16 * kc;
    voff[i] = (4 * va + i) * row_bytes + 16 * vc;
  }
  const uint16_t* kbase = a.k + int64_t(hk) * D;
  const uint16_t* vbase = a.v + int64_t(hk) * D;
  const int v_cl = 2 * (va >> 2) + (va & 1);   // logical 16-byte chunk of keys 4va..4va+3
  const int v_hb = (va >> 1) & 1;              // which 8-byte half of that chunk
  uint4 rk[4], rv[4];

  auto gload = [&](int ka, int k1) {
    // valid bytes: rows ka .. k1-1, 256 bytes of head hk in the last one
    const int bytes = (k1 - ka - 1) * row_bytes + D * 2;
    const int64_t off = int64_t(ka) * a.Hkv * D;
    const __amdgpu_buffer_rsrc_t rsk = make_rsrc(kbase + off, bytes);
    const __amdgpu_buffer_rsrc_t rsv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rk[i] = buf16(rsk, koff[i]);
      rv[i] = buf16(rsv, voff[i]);
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* kb = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(kb + (kr + 16 * i) * K_PITCH + 16 * kc) = rk[i];
    unsigned char* vb = kb + K_BYTES;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t x0 = (&rv[0].x)[m], x1 = (&rv[1].x)[m];
      const uint32_t x2 = (&rv[2].x)[m], x3 = (&rv[3].x)[m];
      // d = 8 vc + 2m (low halves) and d + 1 (high halves); 4 keys each
      const int d0 = 8 * vc + 2 * m;
      const uint2 lo = make_uint2((x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16));
      const uint2 hi = make_uint2((x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u));
      const int sw = (d0 >> 1) & 7;   // same swizzle for rows d0 and d0 + 1
      *reinterpret_cast<uint2*>(vb + d0 * 128 + 16 * (v_cl ^ sw) + 8 * v_hb) = lo;
      *reinterpret_cast<uint2*>(vb + (d0 + 1) * 128 + 16 * (v_cl ^ sw) + 8 * v_hb) = hi;
    }
  };

  int s = it.span0;
  const int s_end = it.span0 + it.nspan;
  pg_key_span sp = a.spans[s];
  int ka = sp.k0;
  gload(ka, sp.k1);
  wait_all_vmem();
  lstore(0);
  __syncthreads();
  int buf = 0;

  while (true) {
    // next tile
    int ns = s, nka = ka + KT;
    pg_key_span nsp = sp;
    if (nka >= sp.k1) {
      ns = s + 1;
      if (ns < s_end) {
        nsp = a.spans[ns];
        nka = nsp.k0;
      }
    }
    const bool has_next = ns < s_end;
    if (has_next) gload(nka, nsp.k1);

    // ---- compute on the current tile ------------------------------------
    const bool is_prefix = sp.k1 <= it.pe;
    bool part = wave_active && ka <= te - 1;
    if (!is_prefix) part = part && (__ballot(row_valid && ss_t == sp.k0) != 0ull);
    if (part) {
      const bool full = (ka + KT <= sp.k1) && (ka + KT - 1 <= tb) && (is_prefix || ss_max <= ka);
      const unsigned char* kb = smem + buf * STAGE;
      f32x16_t sacc[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[0][i] = 0.f;
        sacc[1][i] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const bf16x8_t av = as_bf16x8(
              *reinterpret_cast<const uint4*>(kb + (32 * kb2 + qi) * K_PITCH + 32 * ks + 16 * half));
          sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], sacc[kb2], 0, 0, 0);
        }
      }
      // S^T C-layout: register i of block kb2 holds key 32 kb2 + 8 (i/4) + 4 half + i%4.
      if (!full) {
        // (the empty volatile asm keeps this a real, uniform branch: without
        // it the compiler turns the mask into selects executed on every tile)
        asm volatile("" ::: "memory");
        // allowed keys of this lane's query inside the span: [lo, hi] with
        // lo = own segment start (suffix spans) and hi = min(t, k1 - 1); in
        // tile-local offsets c = 32 kb + 8 (i/4) + i%4 after removing 4 half.
        const int base = ka + 4 * half;
        const int lo = (is_prefix ? ka : ss_t) - base;
        const int hi = min(tq, sp.k1 - 1) - base;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int c = 32 * kb2 + 8 * (i >> 2) + (i & 3);
            sacc[kb2][i] = (c >= lo && c <= hi) ? sacc[kb2][i] : -__builtin_inff();
          }
      }
      float mt = sacc[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sacc[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[1][i]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mt2 = mt * a.c_log2;
      // rescale (wave-uniform decision) only when some row's max grew a lot
      if (__ballot(mt2 > m_run + RESCALE_SLACK) != 0ull) {
        const float m_new = fmaxf(m_run, mt2);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }
      const float m_use = m_run;
      float lsum = 0.f;
      bf16x8_t pf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        uint4 pk;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int i = 8 * (ks & 1) + 2 * jj;
          const float p0 = fast_exp2(fmaf(sacc[ks >> 1][i], a.c_log2, -m_use));
          const float p1 = fast_exp2(fmaf(sacc[ks >> 1][i + 1], a.c_log2, -m_use));
          // the denominator sums the unrounded p in fp32: a sum of the bf16 P
          // would carry bf16's 2^-9 relative error into lse
          lsum += p0 + p1;
          (&pk.x)[jj] = pack_bf16x2(p0, p1);
        }
        pf[ks] = as_bf16x8(pk);
      }
      l_run += lsum;
      const unsigned char* vb = kb + K_BYTES;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8_t av = as_bf16x8(*reinterpret_cast<const uint4*>(
              vb + (32 * db + qi) * 128 + 16 * ((2 * ks + half) ^ ((qi >> 1) & 7))));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[ks], acc[db], 0, 0, 0);
        }
      }
    }

    if (!has_next) break;
    lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    s = ns;
    ka = nka;
    sp = nsp;
  }

  // ---- epilogue -----------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (row_valid) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = a.o + (int64_t(tq) * a.Hq + h) * D;
    // O^T C-layout: register i of block db holds d = 32 db + 8 (i/4) + 4 half + i%4.
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * half;
        const uint2 w = make_uint2(pack_bf16x2(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv),
                                   pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv));
        *reinterpret_cast<uint2*>(orow + d0) = w;
      }
    if (a.lse && half == 0)
      a.lse[int64_t(h) * a.T + tq] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
  }
}

}  // namespace

hipError_t pg_launch_attn_mfma(const pg_layout& L, const void* q, const void* k, const void* v,
                               void* o, float* lse, float softmax_scale, hipStream_t stream) {
  if (L.items.empty()) return hipSuccess;
  MfmaArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.items = L.d_items;
  a.spans = L.d_spans;
  a.tok_ss = L.d_ss;
  a.T = int32_t(L.T);
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.r = L.Hq / L.Hkv;
  a.hpw = L.heads_per_item;
  a.c_log2 = softmax_scale * 1.44269504088896340736f;
  attn_fwd_bf16_d128<<<dim3(uint32_t(L.items.size())), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}
