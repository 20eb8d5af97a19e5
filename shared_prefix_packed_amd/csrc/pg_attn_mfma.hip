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
// Work item (one workgroup of 8 waves): query tokens [t0, t1) of one group and
// `hpw` query heads of one KV head; wave w takes head hq0 + w % hpw and the
// 32-token block w / hpw. All eight waves share every K/V tile staged in LDS,
// so a tile fetched once serves hpw heads (GQA) and every suffix in the block
// (the prefix keys are common to all of them).
//
// Per wave and 64-key tile, with 32x32x16 bf16 MFMAs:
//   S^T[key][query] = K . Q^T     A = K rows from LDS, B = Q from registers
//   online softmax per query      one query per lane, keys split over the two
//                                 lane halves: in-lane max/add + 1 shuffle
//   O^T[d][query]  += V^T . P^T   A = V^T via transposing LDS reads, B = P
//                                 straight from the S^T accumulators
//
// Ping-pong schedule. Softmax costs about as many VALU cycles (one quarter-rate
// exp per score) as the two products cost MFMA cycles, so the two must run at
// the same time. Each wave alternates an MFMA step (PV of the previous tile,
// then S of the current one) with a VALU step (softmax of the current tile).
// Waves 0-3 (group A) run [MFMA; VALU] per tile and waves 4-7 (group B)
// [VALU; MFMA]; waves w and w + 4 share a SIMD, so on each SIMD one wave feeds
// the matrix cores while the other runs the softmax. One workgroup barrier per
// tile keeps the ring consistent (a second one between the steps cost more than
// it brought).
//
// Staging. K and V tiles go from global memory straight into a four-stage LDS
// ring (buffer loads that write LDS, no registers), issued two tiles ahead:
// group A fetches K, group B fetches V. K rows keep their 256 bytes with the
// 16-byte chunks XOR-swizzled by row (conflict-free 128-bit reads). V is stored
// in the order the transposing read ds_read_b64_tr_b16 consumes it: for each
// 16-key step, 8-key half and 32-d block one 512-byte block, in which lane s of
// every 16-lane group owns 8 bytes; one such read then hands each lane 4 keys
// of one d, which is exactly an MFMA A-operand fragment of V^T. The key order
// inside each 16-key step is the one the S^T accumulators give P. A wave
// issues the operand reads of its first two PV products at the end of its
// VALU step, so the MFMA step starts without waiting on LDS.
//
// Output. The normalised O^T tile of each wave goes through LDS once the ring
// is idle, so that O leaves in whole 256-byte rows (16 bytes per lane) rather
// than as 32 scattered 16-byte pieces per store.
#include <hip/hip_runtime.h>

#include "pg_hip_common.h"
#include "pg_internal.h"

namespace {

using namespace pg_hip;

constexpr int D = 128;
constexpr int KT = PG_KEY_TILE;         // 64 keys per tile
constexpr int QW = PG_WAVE_QUERIES;     // 32 queries per wave
constexpr int NWAVES = PG_ITEM_WAVES;   // 8 waves: two groups of 4
constexpr int K_BYTES = KT * D * 2;     // 16384: 64 rows x 256 bytes, swizzled chunks
constexpr int V_BYTES = KT * D * 2;     // 16384: 32 blocks of 512 bytes
constexpr int STAGE = K_BYTES + V_BYTES;
constexpr int NSTAGE = 4;
constexpr int LOADS_PER_TILE = 4;       // 1 KB buffer->LDS loads per wave per tile

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

// The running max is raised only when a tile's max exceeds it by more than
// this many powers of two; until then exp2 arguments stay <= 8 and O, l are
// not rescaled. The result is exact either way: numerator and denominator
// share the same stale max.
constexpr float RESCALE_SLACK = 8.0f;

// s_waitcnt vmcnt(N) (gfx9 encoding: expcnt and lgkmcnt fields left at "no wait").
__device__ inline void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ inline void wait_vmem_but_one_tile() { __builtin_amdgcn_s_waitcnt(0x0F70 | LOADS_PER_TILE); }

// End of a tile: the workgroup barrier alone. Tile fetches and LDS reads may
// stay in flight across it (a __syncthreads() fence would drain both): every
// LDS read is consumed by the step after the one that issued it at the
// latest, and a ring stage is refilled one barrier after its last read. The asm's memory clobber keeps the compiler from moving memory
// operations across; the scheduling barriers keep arithmetic on its side.
__device__ inline void step_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// The fields of a work item the kernel uses (read with scalar loads).
struct Item {
  int t0, t1, hq0, pe, span0, nspan, ntiles, k0, k1;
};

// Walks the 64-key tiles of an item's key spans (all scalar state).
struct TileIter {
  int s, s_end, ka;
  pg_key_span sp;
  // (readfirstlane: keep the state in SGPRs, so spans are read with scalar
  // loads that never wait behind the in-flight tile fetches)
  __device__ void load(const pg_key_span* spans) {
    // the span table is read-only for the kernel: read it through the constant
    // address space so these are scalar loads (lgkmcnt), not vector loads whose
    // vmcnt wait would also drain the tile fetches in flight
    const __attribute__((address_space(4))) int* cs =
        (const __attribute__((address_space(4))) int*)(spans);
    const int idx = 2 * __builtin_amdgcn_readfirstlane(s);
    sp.k0 = __builtin_amdgcn_readfirstlane(cs[idx]);
    sp.k1 = __builtin_amdgcn_readfirstlane(cs[idx + 1]);
    ka = sp.k0;
  }
  __device__ void init(const pg_key_span* spans, int s0, int n) {
    s = __builtin_amdgcn_readfirstlane(s0);
    s_end = __builtin_amdgcn_readfirstlane(s0 + n);
    load(spans);
  }
  __device__ void next(const pg_key_span* spans) {
    ka += KT;
    if (ka >= sp.k1) {
      ++s;
      if (s < s_end) load(spans);
    }
  }
};

__global__ __launch_bounds__(512, 2) void attn_fwd_bf16_d128(MfmaArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * STAGE];

  // the whole item in one scalar load, before the padding test
  Item it;
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
  // every field in hand before the padding test, so that the item costs one
  // scalar load round trip, not one for the test and another after it
  asm volatile("" ::"s"(it.t0), "s"(it.t1), "s"(it.hq0), "s"(it.pe), "s"(it.span0),
               "s"(it.nspan), "s"(it.ntiles), "s"(it.k0), "s"(it.k1), "s"(a.Hkv), "s"(a.hpw),
               "s"(a.r));
  if (it.nspan == 0) return;   // padding of a shorter XCD queue
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int grp = wave >> 2;    // 0: group A, 1: group B (one step later)
  const int wg = wave & 3;      // wave inside its group
  const int qi = lane & 31;     // query column of this lane inside the wave
  const int half = lane >> 5;   // which half of each 16-wide k step the lane feeds
  const int ntiles = __builtin_amdgcn_readfirstlane(it.ntiles);

  const int h = it.hq0 + wave % a.hpw;
  const int hk = it.hq0 / a.r;   // one KV head per item
  const int tb = it.t0 + QW * (wave / a.hpw);
  const int te = min(tb + QW, it.t1);
  const bool wave_active = tb < te;
  const int tq = wave_active ? min(tb + qi, te - 1) : it.t0;   // padded rows repeat the last one
  const bool row_valid = wave_active && (tb + qi < te);

  // ---- staging: per-lane global byte offsets from a tile's first key row ----
  // Wave wg of a group writes LDS blocks 4 wg + i (i = 0..3) of 1 KB each.
  // K block b = rows 4b..4b+3: lane L -> row 4b + L/16, stored chunk L%16,
  //   which holds global chunk (L%16) ^ (row & 15).
  // V block b = 512-byte read blocks 2b, 2b+1 (block index ks*8 + rd*4 + db);
  //   16-byte unit u of a read block holds V[16ks + 8rd + 4(u/16) + (u%8)/2]
  //   [32db + 16((u/8)&1) + 8(u&1) .. +8].
  // Rows past a span's end read as zero (the buffer descriptor ends at the
  // span), so every stage a product reads holds finite values only.
  const int row_bytes = a.Hkv * D * 2;
  int goff[LOADS_PER_TILE];
#pragma unroll
  for (int i = 0; i < LOADS_PER_TILE; ++i) {
    const int b = 4 * wg + i;
    if (grp == 0) {
      const int row = 4 * b + (lane >> 4);
      const int chunk = (lane & 15) ^ (row & 15);
      goff[i] = row * row_bytes + 16 * chunk;
    } else {
      const int rb = 2 * b + (lane >> 5);   // 512-byte read block
      const int ks = rb >> 3, rd = (rb >> 2) & 1, db = rb & 3;
      const int u = lane & 31, g = u >> 3;
      const int key = 16 * ks + 8 * rd + 4 * (g >> 1) + ((u & 7) >> 1);
      const int d0 = 32 * db + 16 * (g & 1) + 8 * (u & 1);
      goff[i] = key * row_bytes + 2 * d0;
    }
  }
  const uint16_t* gbase = (grp == 0 ? a.k : a.v) + int64_t(hk) * D;
  const int region = grp == 0 ? 0 : K_BYTES;
  const uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)smem));

  auto gload = [&](int ka, int k1, int stage) {
    // tile bounds are wave-uniform; say so, or the resource build turns into
    // a per-lane loop around every load
    ka = __builtin_amdgcn_readfirstlane(ka);
    k1 = __builtin_amdgcn_readfirstlane(k1);
    // valid bytes: rows ka .. k1-1, 256 bytes of head hk in the last one
    const int bytes = (k1 - ka - 1) * row_bytes + D * 2;
    const i32x4_t rs = make_rsrc(gbase + int64_t(ka) * a.Hkv * D, bytes);
    const uint32_t dst = lds_base + uint32_t(stage * STAGE + region + 4096 * wg);
#pragma unroll
    for (int i = 0; i < LOADS_PER_TILE; ++i) buf16_to_lds(rs, goff[i], dst + 1024 * i);
  };

  // Prologue. Its memory latencies are the cost of every work item that no
  // other work hides (one workgroup per compute unit), so the first two tile
  // fetches go out first, from the item's own copy of its first span (no span
  // list read before them), and Q and the segment starts are loaded while
  // they are in flight; a single wait covers all of them.
  TileIter ld;
  ld.s = __builtin_amdgcn_readfirstlane(it.span0);
  ld.s_end = __builtin_amdgcn_readfirstlane(it.span0 + it.nspan);
  ld.sp.k0 = __builtin_amdgcn_readfirstlane(it.k0);
  ld.sp.k1 = __builtin_amdgcn_readfirstlane(it.k1);
  ld.ka = ld.sp.k0;
  gload(ld.ka, ld.sp.k1, 0);
  ld.next(a.spans);
  if (ntiles > 1) {
    gload(ld.ka, ld.sp.k1, 1);
    ld.next(a.spans);
  }

  // Q as the B operand of S^T = K Q^T: lane holds d = 16 ks + 8 half + 0..7.
  bf16x8_t qf[8];
  {
    const uint16_t* qrow = a.q + (int64_t(tq) * a.Hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(ldg16(qrow + 16 * ks));
  }
  const int ss_t = a.tok_ss[tq];
  // Segment starts never decrease along a group's row, so the largest among
  // this wave's rows is the last row's: one scalar load, no cross-lane step.
  const int ss_max = ld_scalar(a.tok_ss, wave_active ? te - 1 : it.t0);

  f32x16_t acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m_run = -1.0e30f;   // finite start: exp2(m_run - m_new) is 0, never NaN
  float l_run = 0.f;

  // ---- LDS read offsets --------------------------------------------------
  // S: A operand of block kb, k step ks = K row 32 kb + qi, chunk 2 ks + half,
  //    stored at chunk (2 ks + half) ^ (qi & 15).
  int koff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = qi * 256 + 16 * ((2 * ks + half) ^ (qi & 15));
  // PV: lane reads 8 bytes at 8 * lane of each 512-byte block.
  const int voff = K_BYTES + 8 * lane;

  // The scalar set-up of each fetch (tile bounds, buffer descriptor, LDS
  // destination) is done one step early, in the VALU step, whose scalar unit
  // is idle; the MFMA step then only issues the loads.
  i32x4_t pend_rs = make_rsrc(gbase, 0);
  uint32_t pend_dst = 0;
  auto prep = [&](int tile) {
    const int ka = __builtin_amdgcn_readfirstlane(ld.ka);
    const int k1 = __builtin_amdgcn_readfirstlane(ld.sp.k1);
    const int bytes = (k1 - ka - 1) * row_bytes + D * 2;
    pend_rs = make_rsrc(gbase + int64_t(ka) * a.Hkv * D, bytes);
    pend_dst = lds_base + uint32_t((tile % NSTAGE) * STAGE + region + 4096 * wg);
    ld.next(a.spans);
  };
  if (ntiles > 2) prep(2);
  wait_vmem_all();
  __syncthreads();

  TileIter cp;   // tile of the next S product
  cp.init(a.spans, it.span0, it.nspan);
  f32x16_t sacc[2];
  bf16x8_t pf[4];
  bool s_part = false;   // this wave computed S of the tile now in sacc
  bool p_part = false;   // this wave holds P of the tile awaiting PV
  int v_ka = 0, v_k1 = 0;
  bool v_prefix = true, v_full = true;
  i16x4_t vpre[8];   // first PV operand reads, issued at the end of the VALU step

  // One MFMA step (n) and one VALU step (softmax of tile n), as lambdas; group
  // A runs [M(n); V(n)] and group B [V(n-1); M(n)], so that across a loop back
  // edge only P (group A) or only the S accumulators (group B) stay live.
  auto mfma_step = [&](const int n) {
    // MFMA step n: PV(n-1), S(n), then fetch tile n+2
    __builtin_amdgcn_s_setprio(3);   // the arbiter favours the wave feeding the matrix cores
    if (p_part) {
      const unsigned char* vb = smem + ((n - 1) % NSTAGE) * STAGE + voff;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int j = 4 * ks + db;
          const i16x4_t lo = j < 2 ? vpre[2 * j] : lds_read_tr(vb + 512 * (8 * ks + db));
          const i16x4_t hi = j < 2 ? vpre[2 * j + 1] : lds_read_tr(vb + 512 * (8 * ks + 4 + db));
          const bf16x8_t av = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[ks], acc[db], 0, 0, 0);
        }
      }
      // issue order: 6 reads ahead, then (1 MFMA, 2 reads), so LDS latency
      // hides behind the matrix core instead of stalling it
      sched_reads_ahead<0, 2, 14>();
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    // the K operands of the first S(n) step, read while PV(n-1) runs
    uint4 kpre[2];
    {
      const unsigned char* kbn = smem + (n % NSTAGE) * STAGE;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        kpre[j] = *reinterpret_cast<const uint4*>(kbn + 8192 * (j & 1) + koff[j >> 1]);
    }
    // keep PV(n-1) ahead of S(n): P dies before the S accumulators are born
    __builtin_amdgcn_sched_barrier(0);
    s_part = false;
    if (n < ntiles) {
      const int ka = cp.ka;
      const pg_key_span sp = cp.sp;
      const bool is_prefix = sp.k1 <= it.pe;
      bool part = wave_active && ka <= te - 1;
      if (!is_prefix) part = part && (__ballot(row_valid && ss_t == sp.k0) != 0ull);
      v_ka = ka;
      v_k1 = sp.k1;
      v_prefix = is_prefix;
      v_full = (ka + KT <= sp.k1) && (ka + KT - 1 <= tb) && (is_prefix || ss_max <= ka);
      s_part = part;
      if (part) {
        const unsigned char* kb = smem + (n % NSTAGE) * STAGE;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[0][i] = 0.f;
          sacc[1][i] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            const bf16x8_t av =
                ks < 1 ? as_bf16x8(kpre[2 * ks + kb2])
                       : as_bf16x8(*reinterpret_cast<const uint4*>(kb + 8192 * kb2 + koff[ks]));
            sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], sacc[kb2], 0, 0, 0);
          }
        }
        sched_reads_ahead<0, 1, 14>();
      }
      cp.next(a.spans);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Tile n+2 replaces tile n-2 in the ring; its last readers (PV(n-2) in
    // M(n-1) of both groups) finished before the previous barrier.
    if (n + 2 < ntiles) {
#pragma unroll
      for (int i = 0; i < LOADS_PER_TILE; ++i) buf16_to_lds(pend_rs, goff[i], pend_dst + 1024 * i);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto valu_step = [&](const int n) {
    // VALU step: softmax of tile n (in sacc) -> P
    p_part = s_part;
    if (s_part) {
      // S^T C-layout: register i of block kb holds key 32 kb + 8 (i/4) + 4 half + i%4.
      if (!v_full) {
        // (the empty volatile asm keeps this a real, uniform branch)
        asm volatile("" ::: "memory");
        // allowed keys of this lane's query inside the span: [lo, hi] with
        // lo = own segment start (suffix spans) and hi = min(t, k1 - 1); in
        // tile-local offsets c = 32 kb + 8 (i/4) + i%4 after removing 4 half.
        // The lane's allowed offsets become one 64-bit mask, and each score
        // takes its bit by a signed bitfield extract (0 or -1) and a bitwise
        // select: no compare into VCC per score (each would need wait states
        // before its select). A 32-key block that no lane masks is skipped
        // whole (the diagonal usually cuts only one of the two).
        const int base = v_ka + 4 * half;
        const int lo = (v_prefix ? v_ka : ss_t) - base;
        const int hi = min(tq, v_k1 - 1) - base;
        // bit c of M: tile-local key offset c in [lo, hi]
        const int l0 = max(lo, 0), h0 = min(hi, 63);
        const uint64_t full = ~uint64_t(0);
        const uint64_t M = h0 < l0 ? uint64_t(0) : ((full >> (63 - h0)) & (full << l0));
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const uint32_t w = uint32_t(M >> (32 * kb2));
          if (__ballot((w & 0x0F0F0F0Fu) != 0x0F0F0F0Fu) != 0ull) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int c = 8 * (i >> 2) + (i & 3);
              const int keep = __builtin_amdgcn_sbfe(int(w), c, 1);   // -1 kept, 0 masked
              sacc[kb2][i] = __int_as_float((__float_as_int(sacc[kb2][i]) & keep) |
                                            (int(0xff800000u) & ~keep));
            }
          }
        }
      }
      float mt = sacc[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sacc[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[1][i]);
      {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
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
      // first operand reads of PV(n), used by the next MFMA step: tile n's V
      // was published before an earlier barrier
      const unsigned char* vb = smem + (n % NSTAGE) * STAGE + voff;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        vpre[2 * j] = lds_read_tr(vb + 512 * j);
        vpre[2 * j + 1] = lds_read_tr(vb + 512 * (4 + j));
      }
    }
    s_part = false;
    if (n >= 0 && n + 3 < ntiles) prep(n + 3);   // the fetch of the next MFMA step
  };
  // End of iteration n (both groups have issued M(n)): this wave's part of
  // tile n+1 must have landed before the barrier, since both groups read tile
  // n+1 after it; the fetch of tile n+2 (issued in M(n)) may stay in flight.
  auto end_of_iteration = [&](const int n) {
    if (n + 2 < ntiles)
      wait_vmem_but_one_tile();
    else
      wait_vmem_all();
    step_barrier();
  };

  if (grp == 0) {
    for (int n = 0; n <= ntiles; ++n) {
      mfma_step(n);
      valu_step(n);
      end_of_iteration(n);
    }
  } else {
    for (int n = 0; n <= ntiles; ++n) {
      valu_step(n - 1);
      mfma_step(n);
      end_of_iteration(n);
    }
  }

  // no tile fetch may still be landing in the ring, and no wave still reads it
  wait_vmem_all();
  __syncthreads();

  // ---- epilogue -----------------------------------------------------------
  // O^T C-layout: register i of block db holds d = 32 db + 8 (i/4) + 4 half +
  // i%4 of query column qi. The tile goes through this wave's 8 KB of the
  // (now idle) ring, 16-byte chunks XOR-swizzled by row, so that each store
  // below writes whole 256-byte rows of O.
  const float l_tot = l_run + other_half(l_run);
  const float inv = 1.f / l_tot;
  unsigned char* ot = smem + 8192 * wave;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * half;   // 4 values, 8 bytes
      const uint2 w = make_uint2(pack_bf16x2(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv),
                                 pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv));
      const int chunk = (d0 >> 3) ^ (qi & 15);
      *reinterpret_cast<uint2*>(ot + qi * 256 + 16 * chunk + 8 * half) = w;
    }
  if (wave_active && a.lse && half == 0 && row_valid)
    a.lse[int64_t(h) * a.T + tq] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's tile is in LDS
  if (wave_active) {
    // lane: row 4 it + lane / 16, chunk lane % 16
#pragma unroll
    for (int it2 = 0; it2 < 8; ++it2) {
      const int r = 4 * it2 + (lane >> 4);
      const int c = lane & 15;
      const uint4 v = *reinterpret_cast<const uint4*>(ot + r * 256 + 16 * (c ^ (r & 15)));
      if (tb + r < te)
        *reinterpret_cast<uint4*>(a.o + (int64_t(tb + r) * a.Hq + h) * D + 8 * c) = v;
    }
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
  attn_fwd_bf16_d128<<<dim3(uint32_t(L.items.size())), dim3(64 * NWAVES), 0, stream>>>(a);
  return hipGetLastError();
}
