// Packed shared-prefix attention backward, bf16, d = 128, for gfx950 (CDNA4).
//
// The derivative of the forward (pg_attn_fwd) for an upstream gradient dO, by
// the chain rule: with P the softmax of a query row over its key set K(t),
//   dV = P^T dO,  dS = P * (dO V^T - D),  D = rowsum(dO * O),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// summed over the query heads of each KV head. The prompt is stored once
// ("Preference Packing", core idea), so a prompt key's dK and dV collect the
// gradient of every response of its group. P is recomputed from Q, K and the
// forward's lse, so no attention matrix is kept.
//
// Two launches:
//  * bwd_dq_kernel: the forward's work items (query blocks x heads). Per wave
//    32 query rows. Its prologue works out D of each row from the dO row it
//    loads anyway and writes it out for the next launch. Then per 64-key tile
//    of the item's key spans
//      S^T = K Q^T, dP^T = V dO^T           (A = K, V rows from LDS)
//      P^T = exp2(S^T c - lse2), dS^T = P^T (dP^T - D)
//      dQ^T += K^T dS^T                     (A = K^T by transposing LDS reads,
//                                            B = dS^T from the accumulators)
//    so Q, dO and dQ stay in registers and each key tile is staged once for
//    the eight waves. Waves 4-7 run half a tile behind waves 0-3 (P, dS and
//    the dQ product of the previous tile, then S and dP of this one), so the
//    two waves of a SIMD do not reach the softmax at the same time.
//  * bwd_dkv_kernel: key blocks of at most 128 keys of one KV head inside one
//    segment. The queries that read key j are one contiguous range [j, qend)
//    (the group's end for a prompt key, the response's end otherwise), taken
//    in tiles of 64 rows for each of the r query heads, from the top down: the
//    blocks of one segment share that end, so blocks running side by side on
//    an XCD read the same Q and dO tiles at about the same time. Each 32-key
//    slice is taken by two waves that share a SIMD, each tile in two halves
//    split by the tile's workgroup barrier:
//      dV wave: S = Q K^T, P (to LDS, fp16)  |  dV += P^T dO
//      dK wave: dP = dO V^T, dP - D          |  dS = P (dP - D), dK += dS^T Q
//    (A = Q, dO rows from LDS, B = K, V in registers; A = P^T, dS^T from the
//    accumulators, B = dO, Q by transposing LDS reads; lse and D per query
//    row from LDS). P is computed once per slice and handed over through LDS,
//    so each wave of the pair issues 32 MFMAs per tile; each holds half the
//    operands, which lets two fit on a SIMD; K, V, dK and dV stay in
//    registers for the whole block and no atomics are needed.
// Tiles go HBM -> LDS with buffer loads that write LDS (as in the forward),
// four (dQ, fetched two tiles ahead) or three (dK, dV) stages deep, with one
// workgroup barrier per tile.
#include <hip/hip_runtime.h>

#include "pg_hip_common.h"
#include "pg_internal.h"

namespace {

using namespace pg_hip;

constexpr int D = 128;
constexpr float LOG2E = 1.44269504088896340736f;

// ------------------------------------------------------------------ helpers --

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 4 bytes per lane from buffer `r` at byte offset `voff` into LDS at
// lds + 4 * lane. Same invariant as buf16_to_lds: M0 is written one wait
// state before the load that reads it, and the build's M0 check fails if any
// other instruction of the object touches M0.
__device__ inline void buf4_to_lds(i32x4_t r, int voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(r), "s"(lds)
      : "memory");
}

// Writes a 32 x 128 fp32 tile held as four 32x32 accumulator blocks (block db
// covers d = 32 db .. 32 db + 31), scaled by `mul` and rounded to bf16,
// through LDS region `ot` (8 KB, 16-byte chunks XOR-swizzled by row) to the
// global rows dst + row * row_elems, rows [0, nrows), as whole 256-byte rows.
// ROWS_ARE_REGS: the accumulator rows (register i: row 8 (i/4) + 4 half + i%4)
// are the tile rows and the lanes are d; otherwise the lanes are the tile rows
// and the registers are d.
template <bool ROWS_ARE_REGS>
__device__ inline void store_tile(const f32x16_t* acc, float mul, unsigned char* ot, int lane,
                                  uint16_t* dst, int64_t row_elems, int nrows) {
  const int col = lane & 31, half = lane >> 5;
  if constexpr (!ROWS_ARE_REGS) {
    // lane = tile row (query), registers = d: 4 consecutive d per 8 bytes
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * half;
        const uint2 w = make_uint2(pack_bf16x2(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                                   pack_bf16x2(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul));
        const int chunk = (d0 >> 3) ^ (col & 15);
        *reinterpret_cast<uint2*>(ot + col * 256 + 16 * chunk + 8 * half) = w;
      }
  } else {
    // registers = tile row (key), lane = d: one bf16 per element
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * half + (i & 3);
        const int d = 32 * db + col;
        const int chunk = (d >> 3) ^ (row & 15);
        const __bf16 b = static_cast<__bf16>(acc[db][i] * mul);   // nearest-even
        *reinterpret_cast<__bf16*>(ot + row * 256 + 16 * chunk + 2 * (d & 7)) = b;
      }
  }
  wait_lds();
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = 4 * it + (lane >> 4);
    const int c = lane & 15;
    const uint4 v = *reinterpret_cast<const uint4*>(ot + r * 256 + 16 * (c ^ (r & 15)));
    if (r < nrows) *reinterpret_cast<uint4*>(dst + int64_t(r) * row_elems + 8 * c) = v;
  }
}

// ---------------------------------------------------------------------- dQ --

constexpr int Q_KT = PG_KEY_TILE;            // 64 keys per tile
constexpr int Q_QW = PG_WAVE_QUERIES;        // 32 query rows per wave
constexpr int Q_WAVES = PG_ITEM_WAVES;       // 8 waves, as the forward's items
constexpr int Q_REGION = Q_KT * D * 2;       // 16 KB
constexpr int Q_STAGE = 2 * Q_REGION;        // K, V row-major (K^T by transposing reads of K)
constexpr int Q_NSTAGE = 4;
constexpr int Q_LOADS = 4;                   // 1 KB loads per wave per tile

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const uint16_t* o;
  const float* lse;
  float* delta;   // written by the dQ launch, read by the dK/dV launch
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const pg_work_item* items;
  const pg_key_span* spans;
  const int32_t* tok_ss;
  const pg_kv_item* kv_items;
  int32_t T, Hq, Hkv, r, hpw;
  float c_log2;   // softmax_scale * log2(e)
  float scale;
};

// Walks the 64-key tiles of an item's key spans (scalar state).
struct SpanTiles {
  int s, s_end, ka, k0, k1;
  __device__ void load(const pg_key_span* spans) {
    k0 = ld_scalar(spans, 2 * s);
    k1 = ld_scalar(spans, 2 * s + 1);
    ka = k0;
  }
  __device__ void next(const pg_key_span* spans) {
    ka += Q_KT;
    if (ka >= k1 && ++s < s_end) load(spans);
  }
};

__global__ __launch_bounds__(512, 2) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[Q_NSTAGE * Q_STAGE];

  pg_work_item it;
  {
    const __attribute__((address_space(4))) int* c =
        (const __attribute__((address_space(4))) int*)(a.items + blockIdx.x);
    it.t0 = c[0];
    it.t1 = c[1];
    it.hq0 = c[2];
    it.pe = c[3];
    it.span0 = c[4];
    it.nspan = c[5];
    it.ntiles = c[6];
    it.k0 = c[7];
    it.k1 = c[8];
  }
  asm volatile("" ::"s"(it.t0), "s"(it.t1), "s"(it.hq0), "s"(it.pe), "s"(it.span0),
               "s"(it.nspan), "s"(it.ntiles), "s"(it.k0), "s"(it.k1));
  if (it.nspan == 0) return;   // padding of a shorter XCD queue
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = lane & 31;
  const int half = lane >> 5;

  const bool lag = wave >= 4;
  const int h = it.hq0 + wave % a.hpw;
  const int hk = it.hq0 / a.r;
  const int tb = it.t0 + Q_QW * (wave / a.hpw);
  const int te = min(tb + Q_QW, it.t1);
  const bool wave_active = tb < te;
  const int tq = wave_active ? min(tb + qi, te - 1) : it.t0;
  const bool row_valid = wave_active && (tb + qi < te);

  // staging: waves 0-3 bring K (blocks 4 w + i), waves 4-7 V
  const int w4 = wave & 3;
  const bool vgrp = wave >= 4;
  const int kv_row_bytes = a.Hkv * D * 2;
  int goff[Q_LOADS];
  uint32_t ldst[Q_LOADS];
  const uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)smem));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    goff[i] = rowmajor_off(4 * w4 + i, lane, kv_row_bytes);
    ldst[i] = (vgrp ? Q_REGION : 0) + 1024 * (4 * w4 + i);
  }
  auto fetch = [&](int ka, int k1, int stage) {
    ka = __builtin_amdgcn_readfirstlane(ka);
    k1 = __builtin_amdgcn_readfirstlane(k1);
    const int bytes = (k1 - ka - 1) * kv_row_bytes + D * 2;
    const int64_t row0 = (int64_t(ka) * a.Hkv + hk) * D;
    const i32x4_t rs = make_rsrc((vgrp ? a.v : a.k) + row0, bytes);
    const uint32_t sb = lds_base + uint32_t(stage * Q_STAGE);
#pragma unroll
    for (int i = 0; i < Q_LOADS; ++i) buf16_to_lds(rs, goff[i], sb + ldst[i]);
  };

  // The first two tile fetches go out before anything else, from the item's
  // own copy of its first span (no span-list read before them); Q, dO, lse,
  // the segment starts and O (for D) load while they are in flight.
  const int ntiles = __builtin_amdgcn_readfirstlane(it.ntiles);
  SpanTiles ld;
  ld.s = __builtin_amdgcn_readfirstlane(it.span0);
  ld.s_end = __builtin_amdgcn_readfirstlane(it.span0 + it.nspan);
  ld.k0 = __builtin_amdgcn_readfirstlane(it.k0);
  ld.k1 = __builtin_amdgcn_readfirstlane(it.k1);
  ld.ka = ld.k0;
  for (int n = 0; n < 2 && n < ntiles; ++n) {
    fetch(ld.ka, ld.k1, n);
    ld.next(a.spans);
  }

  // Q and dO rows as B operands (lane: query qi, d = 16 ks + 8 half + 0..7)
  bf16x8_t qf[8], dof[8];
  {
    const int64_t base = (int64_t(tq) * a.Hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = as_bf16x8(ldg16(a.q + base + 16 * ks));
      dof[ks] = as_bf16x8(ldg16(a.dout + base + 16 * ks));
    }
  }
  float lse2 = a.lse[int64_t(h) * a.T + tq] * LOG2E;
  float dlt = 0.f;
  int ss_t = a.tok_ss[tq];
  // Redefine the loaded values by an empty asm: the compiler waits for their
  // loads once, here. Counted inside the tile loop instead, next to the tile
  // fetches it cannot see, its waits would drain every tile in flight.
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(qf[ks]), "+v"(dof[ks]));
  asm volatile("" : "+v"(lse2), "+v"(dlt), "+v"(ss_t));
  const int ss_max = ld_scalar(a.tok_ss, wave_active ? te - 1 : it.t0);


  // A operand reads: row-major K/V row 32 kb + qi, chunk 2 ks + half (swizzled)
  int koff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = qi * 256 + 16 * ((2 * ks + half) ^ rm_swz(qi));
  const TrOffsets tro(lane);

  f32x16_t dqacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  SpanTiles cp;
  cp.s = ld.s_end - it.nspan;
  cp.s_end = ld.s_end;
  cp.k0 = __builtin_amdgcn_readfirstlane(it.k0);
  cp.k1 = __builtin_amdgcn_readfirstlane(it.k1);
  cp.ka = cp.k0;
  // D = sum_d dO O of this row in fp32: each half of the wave holds half of d.
  // The items cover every (token, head) row once, so D is complete for the
  // dK/dV launch that follows. Formed after the first tile fetches are issued,
  // so that the O loads overlap them.
  {
    const int64_t base = (int64_t(tq) * a.Hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 x = ldg16(a.o + base + 16 * ks);
      const uint4 y = __builtin_bit_cast(uint4, dof[ks]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dlt = fmaf(bf16_lo((&x.x)[j]), bf16_lo((&y.x)[j]), dlt);
        dlt = fmaf(bf16_hi((&x.x)[j]), bf16_hi((&y.x)[j]), dlt);
      }
    }
    dlt += other_half(dlt);
    if (row_valid && half == 0) a.delta[int64_t(h) * a.T + tq] = dlt;
  }
  asm volatile("" : "+v"(dlt));

  // Waves 0-3 take each tile whole in its iteration; waves 4-7 run half a tile
  // behind: first P, dS and the dQ product of the previous tile, then S and dP
  // of this one. The two waves of a SIMD (w and w + 4) thus feed the matrix
  // cores and run the softmax at different times instead of together.
  f32x16_t sacc[2], pacc[2];
  bool h_part = false, h_full = true;   // second half pending: tile state
  int h_lo = 0, h_hi = 0, h_stage = 0;

  // MFMA blocks at raised wave priority, the lagging waves (whose iteration is
  // the longer one: both halves meet the other wave's MFMA block) above the
  // leading ones
  auto first_half = [&](const unsigned char* st) {
    if (lag) __builtin_amdgcn_s_setprio(3); else __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sacc[0][i] = 0.f;
      sacc[1][i] = 0.f;
      pacc[0][i] = 0.f;
      pacc[1][i] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t ak = as_bf16x8(*reinterpret_cast<const uint4*>(st + 8192 * kb + koff[ks]));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[ks], sacc[kb], 0, 0, 0);
      }
    sched_reads_ahead<4, 1, 16>();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t av =
            as_bf16x8(*reinterpret_cast<const uint4*>(st + Q_REGION + 8192 * kb + koff[ks]));
        pacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, dof[ks], pacc[kb], 0, 0, 0);
      }
    sched_reads_ahead<4, 1, 16>();
    __builtin_amdgcn_s_setprio(0);
  };
  // P^T and dS^T; register i of block kb holds key ka + 32 kb + 8 (i/4) + 4 half + i%4
  auto second_half = [&](const unsigned char* st, bool full, int lo, int hi) {
    float p[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) p[kb][i] = fast_exp2(fmaf(sacc[kb][i], a.c_log2, -lse2));
    if (!full) {
      asm volatile("" ::: "memory");
      // keys of the tile this lane's row reads: offsets [lo, hi] as a 64-bit
      // mask; each p takes its bit by a signed bitfield extract and an AND
      const int l0 = max(lo, 0), h0 = min(hi, 63);
      const uint64_t ones = ~uint64_t(0);
      const uint64_t M = h0 < l0 ? uint64_t(0) : ((ones >> (63 - h0)) & (ones << l0));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t w = uint32_t(M >> (32 * kb));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int keep = __builtin_amdgcn_sbfe(int(w), 8 * (i >> 2) + (i & 3), 1);
          p[kb][i] = __int_as_float(__float_as_int(p[kb][i]) & keep);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = p[kb][i] * (pacc[kb][i] - dlt);
    bf16x8_t dsf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) dsf[ks] = pack_step(sacc[ks >> 1], ks);
    // dQ^T += K^T dS^T (K^T by transposing reads of the row-major K tile)
    if (lag) __builtin_amdgcn_s_setprio(3); else __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_rowmajor(st, tro, ks, db), dsf[ks],
                                                            dqacc[db], 0, 0, 0);
    sched_reads_ahead<6, 2, 16>();
    __builtin_amdgcn_s_setprio(0);
  };

  // Start of iteration n: tile n landed (tile n + 1 may still be in flight);
  // after the barrier every wave is done with tile n - 2 (the lagging waves
  // finished it in the previous iteration), whose stage tile n + 2 takes.
  // The state of tile n comes back through the references (none past the
  // last tile).
  auto begin_tile = [&](int n, bool& part, bool& full, int& lo, int& hi) {
    if (n + 1 < ntiles)
      wait_vmem<Q_LOADS>();
    else
      wait_vmem<0>();
    bare_barrier();
    if (n + 2 < ntiles) {
      fetch(ld.ka, ld.k1, (n + 2) % Q_NSTAGE);
      ld.next(a.spans);
    }
    part = false;
    full = true;
    lo = hi = 0;
    if (n < ntiles) {
      const int ka = cp.ka, k1 = cp.k1;
      const bool is_prefix = k1 <= it.pe;
      part = wave_active && ka <= te - 1;
      if (!is_prefix) part = part && (__ballot(row_valid && ss_t == cp.k0) != 0ull);
      full = (ka + Q_KT <= k1) && (ka + Q_KT - 1 <= tb) && (is_prefix || ss_max <= ka);
      const int base = ka + 4 * half;
      lo = (is_prefix ? ka : ss_t) - base;
      hi = min(tq, k1 - 1) - base;
      cp.next(a.spans);
    }
  };

  if (!lag) {
    for (int n = 0; n <= ntiles; ++n) {
      bool part, full;
      int lo, hi;
      begin_tile(n, part, full, lo, hi);
      if (part) {
        const unsigned char* st = smem + (n % Q_NSTAGE) * Q_STAGE;
        first_half(st);
        second_half(st, full, lo, hi);
      }
    }
  } else {
    for (int n = 0; n <= ntiles; ++n) {
      bool part, full;
      int lo, hi;
      begin_tile(n, part, full, lo, hi);
      if (h_part) second_half(smem + h_stage * Q_STAGE, h_full, h_lo, h_hi);
      if (part) first_half(smem + (n % Q_NSTAGE) * Q_STAGE);
      h_part = part;
      h_full = full;
      h_lo = lo;
      h_hi = hi;
      h_stage = n % Q_NSTAGE;
    }
  }

  // every wave is done with the ring before it holds the output tiles
  wait_vmem<0>();
  __syncthreads();
  if (wave_active)
    store_tile<false>(dqacc, a.scale, smem + 8192 * wave, lane,
                      a.dq + (int64_t(tb) * a.Hq + h) * D, int64_t(a.Hq) * D, te - tb);
}

// ------------------------------------------------------------------ dK, dV --

constexpr int KV_QT = 64;                    // query rows per tile
constexpr int KV_WAVES = 8;                  // 4 dV waves + 4 dK waves, 32 keys each
constexpr int KV_REGION = KV_QT * D * 2;     // 16 KB
constexpr int KV_ROWS = 2 * KV_REGION;       // Q, dO row-major
constexpr int KV_STAGE = KV_ROWS + 3 * 256;  // + lse, D, and a sink for unused lanes' loads
constexpr int KV_NSTAGE = 3;
constexpr int KV_LOADS = 5;                  // per wave per tile: 4 x 1 KB + one 256 B load

static_assert((KV_WAVES / 2) * 32 == PG_KV_BLOCK, "key block = 4 slices x 32 keys");

// Waves 0-3 and 4-7 take the same four 32-key slices: the first four compute
// dV (S, P, dV += P^T dO), the last four dK (dP, dS = P (dP - D), dK += dS^T Q)
// with the P of their slice's dV wave. Each role runs its own loop and holds
// only its own operands and accumulators, so two waves fit on a SIMD (waves w
// and w + 4 share one) and hide each other's latency. Both loops take the
// same barrier, one per tile, between the two halves of a tile: P of the
// tile is in LDS and the next tile's stage has landed.
struct KvCtx {
  const pg_kv_item* it;
  int lane, wave, col, half, hk, kw0, kw1, key, q_start, nq, ntiles, q_row_bytes;
  bool wave_keys;
  uint32_t lds_base;
  int goff[2];
};

// tile n = (query tile nq - 1 - n / r from the top down, head hk * r + n % r)
__device__ inline void kv_fetch(const BwdArgs& a, const KvCtx& c, int nt, int nh, int stage) {
  const int m = c.nq - 1 - nt, h = c.hk * a.r + nh;
  const int q0 = c.q_start + KV_QT * m;
  const int rows = min(KV_QT, c.it->qend - q0);
  const int bytes = (rows - 1) * c.q_row_bytes + D * 2;
  const int64_t row0 = (int64_t(q0) * a.Hq + h) * D;
  const i32x4_t rq = make_rsrc(a.q + row0, bytes);
  const i32x4_t rd = make_rsrc(a.dout + row0, bytes);
  const uint32_t sb = c.lds_base + uint32_t(stage * KV_STAGE) + 2048 * c.wave;
#pragma unroll
  for (int i = 0; i < 2; ++i) buf16_to_lds(rq, c.goff[i], sb + 1024 * i);
#pragma unroll
  for (int i = 0; i < 2; ++i) buf16_to_lds(rd, c.goff[i], sb + KV_REGION + 1024 * i);
  // lse (wave 0) or D (wave 1) of the tile's rows; the other waves load
  // nothing into the sink, so that every wave waits for the same count
  const float* src = c.wave == 0 ? a.lse : a.delta;
  const i32x4_t rl = make_rsrc(src + int64_t(h) * a.T + q0, c.wave < 2 ? 4 * rows : 0);
  buf4_to_lds(rl, 4 * c.lane, c.lds_base + uint32_t(stage * KV_STAGE) + KV_ROWS + 256 * min(c.wave, 2));
}

// P of one (query tile, slice) in fp16, as the dV waves hand it to the dK
// waves: the four values of accumulator group m (= 4 kb + g) of lane l at
// byte 512 m + 8 l of the slice's 4 KB; two buffers, for even and odd tiles.
constexpr int KV_PX = KV_NSTAGE * KV_STAGE;
constexpr int KV_PBUF = 4 * 4096;
constexpr int KV_SMEM = KV_PX + 2 * KV_PBUF;

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// nearest-even fp32 -> fp16 of two values (one v_cvt_pk_f16_f32)
__device__ inline uint32_t pack_f16x2(float a, float b) {
  f16x2_t v;
  v.x = static_cast<_Float16>(a);
  v.y = static_cast<_Float16>(b);
  return __builtin_bit_cast(uint32_t, v);
}

// P = exp(S scale - lse) of the 64 x 32 tile in the accumulator layout, zero
// where the row cannot read the key (only on tiles crossing the diagonal or
// the item's last query row).
template <bool MASK>
__device__ inline void tile_p(f32x16_t (&s)[2], const float4 (&l4)[8], float c_log2, int q0,
                              int half, int key, int qend) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g + j;
        float p = fast_exp2(fmaf(s[kb][i], c_log2, -(&l4[4 * kb + g].x)[j] * LOG2E));
        if constexpr (MASK) {
          const int qrow = q0 + 32 * kb + 8 * g + 4 * half + j;
          p = ((qrow >= key) & (qrow < qend)) ? p : 0.f;
        }
        s[kb][i] = p;
      }
}

template <bool KWAVE>
__device__ inline void kv_loop(const BwdArgs& a, const KvCtx& c, unsigned char* smem) {
  const pg_kv_item& it = *c.it;
  // B operands of the first product, rows of the slice's keys (lane: key col,
  // d = 16 ks + 8 half + 0..7; keys past the block are zero): K for S = Q K^T
  // (dV role), V for dP = dO V^T (dK role)
  // The first tile is fetched while these registers load; the second after
  // their wait, which would otherwise drain it as well.
  // (n / r, n % r) of the next tile to fetch, kept as counters
  int ft = 0, fh = 0;
  auto fetch_next = [&](int stage) {
    kv_fetch(a, c, ft, fh, stage);
    if (++fh == a.r) {
      fh = 0;
      ++ft;
    }
  };
  fetch_next(0);
  bf16x8_t bf[8];
  {
    const bool key_valid = c.key < c.kw1;
    const uint16_t* src = KWAVE ? a.v : a.k;
    const int64_t base = (int64_t(key_valid ? c.key : it.k0) * a.Hkv + c.hk) * D + 8 * c.half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      bf[ks] = as_bf16x8(key_valid ? ldg16(src + base + 16 * ks) : make_uint4(0, 0, 0, 0));
    // waited for once, here, not inside the tile loop (see bwd_dq_kernel)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(bf[ks]));
  }
  // A operand reads of row-major Q / dO: row 32 kb + col, chunk 2 ks + half
  int aoff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) aoff[ks] = c.col * 256 + 16 * ((2 * ks + c.half) ^ rm_swz(c.col));
  const TrOffsets tro(c.lane);
  uint2* const px = reinterpret_cast<uint2*>(smem + KV_PX + 4096 * (c.wave & 3)) + c.lane;

  f32x16_t acc[4];   // dV or dK: rows = keys (registers), lanes = d
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  if (c.ntiles > 1) {
    fetch_next(1);
    wait_vmem<KV_LOADS>();
  } else {
    wait_vmem<0>();
  }
  bare_barrier();   // tile 0 has landed

  int lt = 0, lh = 0;   // (n / r, n % r) of this tile
  for (int n = 0; n < c.ntiles; ++n) {
    uint2* const pb = px + (n & 1) * (KV_PBUF / 8);
    const int q0 = c.q_start + KV_QT * (c.nq - 1 - lt);
    if (++lh == a.r) {
      lh = 0;
      ++lt;
    }
    // the slice has keys, and some row of the tile can read one of them
    const bool active = c.wave_keys && q0 + KV_QT - 1 >= c.kw0;
    const unsigned char* st = smem + (n % KV_NSTAGE) * KV_STAGE;

    // first half: S and P (dV role; P goes to LDS), dP - D (dK role)
    f32x16_t sacc[2];
    if (active) {
      // MFMA blocks run at raised wave priority: the arbiter then favours
      // whichever wave of the SIMD is feeding the matrix cores, the dK role
      // (the longer of the two per tile) above the dV role
      __builtin_amdgcn_s_setprio(KWAVE ? 3 : 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[0][i] = 0.f;
        sacc[1][i] = 0.f;
      }
      const unsigned char* at = st + (KWAVE ? KV_REGION : 0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8_t av = as_bf16x8(*reinterpret_cast<const uint4*>(at + 8192 * kb + aoff[ks]));
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bf[ks], sacc[kb], 0, 0, 0);
        }
      sched_reads_ahead<6, 1, 16>();
      __builtin_amdgcn_s_setprio(0);
      // lse (dV role) or D (dK role) of rows 32 kb + 8 g + 4 half + 0..3
      const float* rowv = reinterpret_cast<const float*>(st + KV_ROWS + (KWAVE ? 256 : 0));
      float4 r4[8];
#pragma unroll
      for (int m = 0; m < 8; ++m)
        r4[m] = *reinterpret_cast<const float4*>(rowv + 32 * (m >> 2) + 8 * (m & 3) + 4 * c.half);
      if constexpr (!KWAVE) {
        const bool full = (q0 >= c.kw0 + 31) && (q0 + KV_QT <= it.qend);
        if (full)
          tile_p<false>(sacc, r4, a.c_log2, q0, c.half, c.key, it.qend);
        else
          tile_p<true>(sacc, r4, a.c_log2, q0, c.half, c.key, it.qend);
#pragma unroll
        for (int m = 0; m < 8; ++m)
          pb[64 * m] = make_uint2(pack_f16x2(sacc[m >> 2][4 * (m & 3)], sacc[m >> 2][4 * (m & 3) + 1]),
                                  pack_f16x2(sacc[m >> 2][4 * (m & 3) + 2], sacc[m >> 2][4 * (m & 3) + 3]));
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) sacc[m >> 2][4 * (m & 3) + j] -= (&r4[m].x)[j];
      }
    }
    // One barrier per tile. Before it: this wave's part of tile n + 1 has
    // landed (the only fetch in flight) and the dV wave's P is in LDS. After
    // it, tile n + 2 goes to the stage of tile n - 1, whose last reads (the
    // second half of n - 1) came before this barrier; P of tile n + 1 goes to
    // the other buffer while the dK waves still read this one.
    wait_vmem<0>();
    if constexpr (!KWAVE) wait_lds();
    bare_barrier();
    // the dK role's P reads go out before the fetch, so that their latency
    // overlaps its issue
    uint2 pr[8];
    if constexpr (KWAVE) {
      if (active) {
#pragma unroll
        for (int m = 0; m < 8; ++m) pr[m] = pb[64 * m];
      }
    }
    if (n + 2 < c.ntiles) fetch_next((n + 2) % KV_NSTAGE);
    if (!active) continue;

    // second half: dV += P^T dO, or dS = P (dP - D) and dK += dS^T Q (B by
    // transposing reads of the row-major dO / Q tile)
    if constexpr (KWAVE) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint2 p2 = pr[m];
        const f16x2_t lo = __builtin_bit_cast(f16x2_t, p2.x);
        const f16x2_t hi = __builtin_bit_cast(f16x2_t, p2.y);
        const float p4[4] = {float(lo.x), float(lo.y), float(hi.x), float(hi.y)};
        // fma with a zero addend: one v_fma_mix_f32 straight from the fp16 P
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc[m >> 2][4 * (m & 3) + j] = __builtin_fmaf(p4[j], sacc[m >> 2][4 * (m & 3) + j], 0.f);
      }
    }
    const unsigned char* bt = st + (KWAVE ? 0 : KV_REGION);
    __builtin_amdgcn_s_setprio(KWAVE ? 3 : 1);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const bf16x8_t pf = pack_step(sacc[s2 >> 1], s2);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf, tr_rowmajor(bt, tro, s2, db), acc[db], 0, 0, 0);
    }
    sched_reads_ahead<6, 2, 16>();
    __builtin_amdgcn_s_setprio(0);
  }

  wait_vmem<0>();
  __syncthreads();
  if (c.wave_keys) {
    unsigned char* ot = smem + 8192 * c.wave;
    const int64_t rs = int64_t(a.Hkv) * D;
    uint16_t* dst = (KWAVE ? a.dk : a.dv) + (int64_t(c.kw0) * a.Hkv + c.hk) * D;
    store_tile<true>(acc, KWAVE ? a.scale : 1.f, ot, c.lane, dst, rs, c.kw1 - c.kw0);
  }
}

__global__ __launch_bounds__(512, 1) void bwd_dkv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[KV_SMEM];

  const pg_kv_item it = a.kv_items[blockIdx.x];
  if (it.k1 <= it.k0) return;   // padding
  KvCtx c;
  c.it = &it;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.col = c.lane & 31;
  c.half = c.lane >> 5;
  c.hk = it.hk;
  c.kw0 = it.k0 + 32 * (c.wave & 3);
  c.kw1 = min(c.kw0 + 32, it.k1);
  c.wave_keys = c.kw0 < c.kw1;
  c.key = c.kw0 + c.col;
  c.q_start = it.k0;
  c.nq = (it.qend - c.q_start + KV_QT - 1) / KV_QT;
  c.ntiles = c.nq * a.r;
  c.q_row_bytes = a.Hq * D * 2;
  // staging: wave w brings blocks 2 w, 2 w + 1 of the row-major Q and dO tiles
  c.lds_base = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)smem));
#pragma unroll
  for (int i = 0; i < 2; ++i) c.goff[i] = rowmajor_off(2 * c.wave + i, c.lane, c.q_row_bytes);
  if (c.wave >= 4)
    kv_loop<true>(a, c, smem);
  else
    kv_loop<false>(a, c, smem);
}

}  // namespace

hipError_t pg_launch_attn_bwd(const pg_layout& L, const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const void* dout, void* dq,
                              void* dk, void* dv, float* delta, float softmax_scale,
                              hipStream_t stream) {
  if (L.items.empty()) return hipSuccess;
  BwdArgs a;
  a.o = static_cast<const uint16_t*>(o);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.delta = delta;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.items = L.d_items;
  a.spans = L.d_spans;
  a.tok_ss = L.d_ss;
  a.kv_items = L.d_kv_items;
  a.T = int32_t(L.T);
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.r = L.Hq / L.Hkv;
  a.hpw = L.heads_per_item;
  a.c_log2 = softmax_scale * LOG2E;
  a.scale = softmax_scale;
  bwd_dq_kernel<<<dim3(uint32_t(L.items.size())), dim3(64 * Q_WAVES), 0, stream>>>(a);
  if (!L.kv_items.empty())
    bwd_dkv_kernel<<<dim3(uint32_t(L.kv_items.size())), dim3(64 * KV_WAVES), 0, stream>>>(a);
  return hipGetLastError();
}
