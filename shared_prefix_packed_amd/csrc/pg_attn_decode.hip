// Decode-time shared-prefix attention over a group-contiguous KV cache, bf16,
// d = 128, for gfx950 (CDNA4).
//
// One decode step: the newest token of every response attends to its group's
// prompt rows and its own valid rows (PackInfer abstract, I/O-aware grouping:
// requests that share a prefix are co-located and their KV cache is kept
// group-contiguous while generation proceeds). The work is HBM-bound -- each
// cache row is used by at most n * r query rows -- so the design goal is to
// read every prompt row once per step for the whole group, and every response
// row once, with enough bytes in flight to keep HBM busy:
//
//  * decode_partial_kernel: one wave per work item (host-built, launch order,
//    XCD-balanced): up to 512 cache rows (1024 in a prompt longer than 4096
//    rows) of one KV head inside one segment, for
//    up to 32 query rows (the responses of a group for a prompt chunk, one
//    response for a response chunk). Inside an item every query row sees every
//    key, so there is no per-row mask; a response chunk stops at the
//    response's current length. Tiles of 32 rows of K and V go HBM -> LDS
//    (buffer loads that write LDS, 3-stage ring, two tiles in flight),
//      S^T = K Q^T        (A = K rows from LDS, B = Q held in registers)
//      O^T += V^T P^T     (A = V^T by transposing LDS reads of the row-major
//                          tile, B = P^T straight from the S^T accumulators)
//    with an online softmax in base 2; the unnormalised O^T, the running max
//    and the row sum go to the workspace as the item's partial result.
//  * decode_merge_kernel: one wave per (response, query head) combines the
//    partials of the items holding its row (O = sum e^(m_i - M) O_i / sum
//    e^(m_i - M) l_i) and writes O (bf16) and lse; the partials are fetched
//    side by side, one lane each, rather than one after another.
#include <mutex>

#include "pg_hip_common.h"
#include "pg_internal.h"

namespace {

using namespace pg_hip;

constexpr int D = 128;
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float LN2 = 0.69314718055994530942f;
constexpr int DEC_KT = 32;                     // cache rows per tile
constexpr int DEC_REGION = DEC_KT * D * 2;     // 8 KB: one tile of K or of V
constexpr int DEC_STAGE = 2 * DEC_REGION;      // K then V, row-major, swizzled
constexpr int DEC_NSTAGE = 3;
constexpr int DEC_BLOCKS = DEC_REGION / 1024;  // 1 KB loads per region
constexpr int DEC_LOADS = 2 * DEC_BLOCKS;      // per tile
static_assert(PG_DEC_CHUNK % DEC_KT == 0, "chunks are whole tiles");

struct DecArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* cur_lens;
  const pg_dec_item* items;
  float* ws_o;    // [items][32][D] unnormalised O rows
  float* ws_ml;   // [items][32][2] running max (base 2, scaled) and row sum
  int32_t Hq, Hkv, r;
  float c_log2;   // softmax_scale * log2(e)
};

__global__ __launch_bounds__(64) void decode_partial_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[DEC_NSTAGE * DEC_STAGE];

  const pg_dec_item it = a.items[blockIdx.x];
  if (it.nrow == 0) return;   // padding of a shorter XCD queue
  const int lane = threadIdx.x;
  const int qi = lane & 31;
  const int half = lane >> 5;

  int k1 = it.k1;
  if (it.resp >= 0) {
    const int len = min(max(ld_scalar(a.cur_lens, it.resp), 0), it.seg1 - it.seg0);
    k1 = min(k1, it.seg0 + len);
  }
  const int nkeys = __builtin_amdgcn_readfirstlane(max(k1 - it.k0, 0));
  float* wo = a.ws_o + int64_t(blockIdx.x) * PG_DEC_ROWS * D;
  float* wml = a.ws_ml + int64_t(blockIdx.x) * PG_DEC_ROWS * 2;
  const bool row_valid = qi < it.nrow;
  if (nkeys == 0) {   // a response chunk past the current length
    if (half == 0 && row_valid)
      *reinterpret_cast<float2*>(wml + 2 * qi) = make_float2(-INFINITY, 0.f);
    return;
  }

  // Q rows as B operands (lane: query row qi, d = 16 ks + 8 half + 0..7)
  const int row = it.row0 + min(qi, it.nrow - 1);
  const int kq = row / a.r;
  const int h = it.hk * a.r + (row - kq * a.r);
  bf16x8_t qf[8];
  {
    const int64_t base = (int64_t(kq) * a.Hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(ldg16(a.q + base + 16 * ks));
    // Redefine Q by an empty asm: the compiler waits for the loads once, here,
    // instead of counting them inside the tile loop, where the tile fetches it
    // cannot see would turn its waits into waits for every tile in flight.
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(qf[ks]));
  }

  const int ntiles = (nkeys + DEC_KT - 1) / DEC_KT;
  const int kv_row_bytes = a.Hkv * D * 2;
  int goff[DEC_BLOCKS];
#pragma unroll
  for (int b = 0; b < DEC_BLOCKS; ++b) goff[b] = rowmajor_off(b, lane, kv_row_bytes);
  const uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)smem));
  auto fetch = [&](int n) {
    const int ka = it.k0 + DEC_KT * n;
    const int rows = min(DEC_KT, k1 - ka);
    const int bytes = (rows - 1) * kv_row_bytes + D * 2;   // rows past the end read as zero
    const int64_t row0 = (int64_t(ka) * a.Hkv + it.hk) * D;
    const i32x4_t rk = make_rsrc(a.k + row0, bytes);
    const i32x4_t rv = make_rsrc(a.v + row0, bytes);
    const uint32_t sb = lds_base + uint32_t((n % DEC_NSTAGE) * DEC_STAGE);
#pragma unroll
    for (int b = 0; b < DEC_BLOCKS; ++b) buf16_to_lds(rk, goff[b], sb + 1024 * b);
#pragma unroll
    for (int b = 0; b < DEC_BLOCKS; ++b) buf16_to_lds(rv, goff[b], sb + DEC_REGION + 1024 * b);
  };

  // A operand reads of K: row qi, stored chunk (2 ks + half) ^ rm_swz(qi)
  int koff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = qi * 256 + 16 * ((2 * ks + half) ^ rm_swz(qi));
  const TrOffsets tro(lane);

  f32x16_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int n = 0; n < DEC_NSTAGE - 1 && n < ntiles; ++n) fetch(n);

  for (int n = 0; n < ntiles; ++n) {
    if (n + DEC_NSTAGE - 1 < ntiles) fetch(n + DEC_NSTAGE - 1);
    // tile n landed once at most the loads of the tiles after it are pending
    const int ahead = min(ntiles - 1 - n, DEC_NSTAGE - 1);
    if (ahead == 2)
      wait_vmem<2 * DEC_LOADS>();
    else if (ahead == 1)
      wait_vmem<DEC_LOADS>();
    else
      wait_vmem<0>();
    const unsigned char* st = smem + (n % DEC_NSTAGE) * DEC_STAGE;

    f32x16_t sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t ak = as_bf16x8(*reinterpret_cast<const uint4*>(st + koff[ks]));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[ks], sacc, 0, 0, 0);
    }

    // register i holds key 8 (i/4) + 4 half + i%4 of the tile for query row qi
    const int valid = nkeys - DEC_KT * n;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = 8 * (i >> 2) + 4 * half + (i & 3);
      const float x = kr < valid ? sacc[i] * a.c_log2 : -INFINITY;
      sacc[i] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, other_half(mx));
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(sacc[i] - mn);
      sacc[i] = p;
      ps += p;
    }
    l = l * alpha + ps;
    m = mn;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // O^T += V^T P^T over the tile's two 16-row steps
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8_t pf = pack_step(sacc, s);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_rowmajor(st + DEC_REGION, tro, s, db),
                                                           pf, oacc[db], 0, 0, 0);
    }
    // the stage is refilled by the fetch at the top of iteration n + 1: its
    // reads must have returned first
    wait_lds();
  }

  const float lt = l + other_half(l);
  if (row_valid) {
    if (half == 0) *reinterpret_cast<float2*>(wml + 2 * qi) = make_float2(m, lt);
    // O^T register i of block db: d = 32 db + 8 (i/4) + 4 half + i%4
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(wo + qi * D + 32 * db + 8 * g + 4 * half) =
            make_float4(oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]);
  }
}

// One wave per output row (response k, query head h). The lanes first take
// up to 64 of the row's partials at once (merge-list entry, item, then its
// (m, l): three dependent loads for all of them together), the wave reduces
// the common max M and the weights e^(m_i - M); then every lane sums its 2
// values of d over the partials, eight row loads in flight at a time.
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
    const pg_dec_item* __restrict__ items, const int32_t* __restrict__ ref_off,
    const int32_t* __restrict__ refs, uint16_t* __restrict__ o, float* __restrict__ lse, int32_t N,
    int32_t Hq, int32_t Hkv, int32_t r) {
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= int64_t(N) * Hq) return;
  const int k = int(row / Hq), h = int(row % Hq);
  const int hk = h / r;
  const int qrow = k * r + (h - hk * r);
  float M = -INFINITY, L = 0.f, acc0 = 0.f, acc1 = 0.f;
  const int j0 = ref_off ? ref_off[int64_t(k) * Hkv + hk] : 0;
  const int j1 = ref_off ? ref_off[int64_t(k) * Hkv + hk + 1] : 0;
  for (int jb = j0; jb < j1; jb += 64) {
    const int nb = min(64, j1 - jb);
    // lane j: partial jb + j (slot 0 of item 0 stands in for lanes without one)
    int slot = 0;   // items * 32 fits in 32 bits (T < 2^30 rows)
    float m = -INFINITY, l = 0.f;
    if (lane < nb) {
      const int idx = refs[jb + lane];
      const int row0 = items[idx].row0, nrow = items[idx].nrow;
      if (qrow >= row0 && qrow < row0 + nrow) {
        slot = idx * PG_DEC_ROWS + (qrow - row0);
        const float2 ml = *reinterpret_cast<const float2*>(ws_ml + 2 * int64_t(slot));
        if (ml.y > 0.f) {   // else no key of the item is valid for this row
          m = ml.x;
          l = ml.y;
        }
      }
    }
    float mb = m;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mb = fmaxf(mb, __shfl_xor(mb, off, 64));
    if (mb == -INFINITY) continue;
    const float mn = fmaxf(M, mb);
    const float a0 = exp2f(M - mn);
    const float wgt = l > 0.f ? exp2f(m - mn) : 0.f;
    float lb = wgt * l;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lb += __shfl_xor(lb, off, 64);
    L = L * a0 + lb;
    acc0 *= a0;
    acc1 *= a0;
    M = mn;
    for (int j = 0; j < nb; j += 8) {
      float2 ov[8];
      float wj[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int src = min(j + u, nb - 1);   // wave-uniform
        const float wsrc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), src));
        wj[u] = j + u < nb ? wsrc : 0.f;
        const int64_t sl = __builtin_amdgcn_readlane(slot, src);
        ov[u] = *reinterpret_cast<const float2*>(ws_o + sl * D + 2 * lane);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (wj[u] != 0.f) {   // skip weight-0 partials: their O rows may hold anything
          acc0 = fmaf(wj[u], ov[u].x, acc0);
          acc1 = fmaf(wj[u], ov[u].y, acc1);
        }
      }
    }
  }
  const bool any = L > 0.f;
  const float inv = any ? 1.f / L : 0.f;
  *reinterpret_cast<uint32_t*>(o + row * D + 2 * lane) = pack_bf16x2(acc0 * inv, acc1 * inv);
  if (lane == 0) lse[int64_t(h) * N + k] = any ? (M + log2f(L)) * LN2 : -INFINITY;
}

}  // namespace

size_t pg_decode_workspace_bytes(const pg_layout& L) {
  return L.dec_items.size() * size_t(PG_DEC_ROWS) * size_t(L.d + 2) * sizeof(float);
}

hipError_t pg_launch_attn_decode(const pg_layout& L, const void* q, const void* k, const void* v,
                                 const int32_t* cur_lens, void* o, float* lse, void* workspace,
                                 pg_dtype dtype, float softmax_scale, hipStream_t stream) {
  if (dtype != PG_BF16 || L.d != D)
    return pg_launch_decode_rowwise(L, q, k, v, cur_lens, o, lse, dtype, softmax_scale, stream);
  const int32_t N = int32_t(L.suffix_lens.size());
  const int32_t r = L.Hq / L.Hkv;
  const int64_t nitems = int64_t(L.dec_items.size());
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o ? ws_o + nitems * PG_DEC_ROWS * D : nullptr;
  const bool tables = L.T > 0 && L.d_dec_ref_off != nullptr;
  if (tables && nitems > 0) {
    DecArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.cur_lens = cur_lens;
    a.items = L.d_dec_items;
    a.ws_o = ws_o;
    a.ws_ml = ws_ml;
    a.Hq = L.Hq;
    a.Hkv = L.Hkv;
    a.r = r;
    a.c_log2 = softmax_scale * LOG2E;
    decode_partial_kernel<<<dim3(uint32_t(nitems)), dim3(64), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t rows = int64_t(N) * L.Hq;
  decode_merge_kernel<<<dim3(uint32_t((rows + 3) / 4)), dim3(256), 0, stream>>>(
      ws_o, ws_ml, tables ? L.d_dec_items : nullptr, tables ? L.d_dec_ref_off : nullptr,
      tables ? L.d_dec_refs : nullptr, static_cast<uint16_t*>(o), lse, N, L.Hq, L.Hkv, r);
  return hipGetLastError();
}

// ------------------------------------------------- decode without a workspace --
//
// For callers that cannot allocate device memory, the partial results can live
// in a static device array instead of a caller workspace. Each GPU the library
// runs on holds its own copy until the process ends. In host code the array's
// name is only a stand-in for the device copy: its device address is looked up
// once per device with hipGetSymbolAddress (the device current) and only that
// address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[PG_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t pg_decode_scratch(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}
