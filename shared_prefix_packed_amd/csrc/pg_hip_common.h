// Device helpers shared by the attention kernels of libpg.so (forward,
// backward, decode): operand types, buffer->LDS loads, transposing LDS reads,
// bf16 packing, wait counters, MFMA/LDS-read scheduling patterns and the
// row-major swizzled tile addressing. gfx950 only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pg_hip {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource (four SGPRs) over `bytes` bytes from `base`: 48-bit base,
// stride 0, num_records = bytes, gfx9 dword3 = untyped 32-bit data. Loads at
// or past `bytes` return zeros, so rows past the end of a key span need no
// clamping. Every field must be wave-uniform.
__device__ inline i32x4_t make_rsrc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane(int(uint32_t(p)));
  r[1] = __builtin_amdgcn_readfirstlane(int(uint32_t(p >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from buffer `r` at byte offset `voff` straight into LDS at
// byte address lds + 16 * lane (lds is wave-uniform). Written as asm so the
// compiler does not guard later LDS reads with full vmcnt(0) waits: the loads
// only write LDS (no VGPR result), and their completion is awaited explicitly
// (wait_vmem_*) before the barrier that publishes the tile. With the builtin
// __builtin_amdgcn_raw_ptr_buffer_load_lds the compiler owns M0 but cannot
// tell the ring stages apart, and waits for every load in flight before LDS
// reads (six more vmcnt(0) waits in the forward's tile loop), which drains
// the tiles fetched ahead.
// Invariant: M0 is written here, one wait state before the load that reads
// it, and the compiler cannot be told so (M0 is not accepted in a clobber
// list). This is safe only while no compiler-generated code in these kernels
// uses M0; the build (build.py, check_m0) disassembles every HIP object and
// fails if any instruction other than these sequences touches M0.
__device__ inline void buf16_to_lds(i32x4_t r, int voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(r), "s"(lds)
      : "memory");
}

__device__ inline bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Transposing LDS read: inside each group of 16 lanes, lane d receives element
// d % 4 of the 8-byte chunks addressed by lanes 4 j + d / 4, j = 0..3.
__device__ inline i16x4_t lds_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  // nearest-even fp32 -> bf16 of two values in one v_cvt_pk_bf16_f32
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane l ^ 32 (the other half of the wave), through a VALU lane swap
// instead of an LDS round trip.
__device__ inline float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0] holds lanes 0-31 in both halves, r[1] lanes 32-63 in both halves
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Wave-uniform int from read-only global memory, as a scalar load.
__device__ inline int ld_scalar(const void* base, int i) {
  const __attribute__((address_space(4))) int* c = (const __attribute__((address_space(4))) int*)(base);
  return __builtin_amdgcn_readfirstlane(c[i]);
}

// s_waitcnt vmcnt(N) for N < 64 (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt and lgkmcnt fields left at "no wait").
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// s_waitcnt lgkmcnt(0) (vmcnt and expcnt fields at "no wait").
__device__ inline void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier alone (no memory fence: loads may stay in flight). The
// memory clobber keeps the compiler from moving memory operations across; the
// scheduling barriers keep arithmetic on its side.
__device__ inline void bare_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Scheduling pattern for a block of NM MFMAs fed by LDS reads: AHEAD reads
// first, then PER reads after each MFMA until the reads run out.
template <int I, int NM, int PER, int REST>
__device__ inline void sched_mfma_then_reads() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    constexpr int r = REST >= PER ? PER : REST;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);   // r LDS reads
    sched_mfma_then_reads<I + 1, NM, PER, REST - r>();
  }
}
template <int AHEAD, int PER, int NM>
__device__ inline void sched_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
  sched_mfma_then_reads<0, NM, PER, NM * PER - AHEAD>();
}

// Rotate-half RoPE of the pair (x_i, x_{i+d/2}) = (xl, xh) by the angle with
// cosine c and sine s, in fp64 with explicit fused multiply-adds, so every
// kernel that rotates gets the same bits.
__device__ inline double rope_lo(double xl, double xh, double c, double s) {
  return __fma_rn(xl, c, -(xh * s));
}
__device__ inline double rope_hi(double xl, double xh, double c, double s) {
  return __fma_rn(xh, c, xl * s);
}

// ------------------------------------------- row-major tiles of 256-byte rows --

// Chunk swizzle of a row-major tile (256-byte rows, sixteen 16-byte chunks):
// global chunk c of row r sits at chunk c ^ swz(r), swz(r) the 4-bit rotation
// of r % 16, ((r & 3) << 2) | ((r & 15) >> 2). A plain c ^ (r % 16) spreads
// row-wise reads over all 64 banks too, but keeps the eight rows of a
// transposing read (below) on two 4-chunk groups, 32 banks: twice the cycles.
// The rotation gives those rows all four groups, and it is still a bijection
// of r % 16, so row-wise reads of 16 consecutive rows stay conflict-free.
__device__ inline int rm_swz(int row) {
  const int r = row & 15;
  return ((r & 3) << 2) | (r >> 2);
}

// Byte offset (from a tile's first row) of the 16-byte global unit that lane
// `lane` of 1 KB block `b` brings into a row-major tile: row 4 b + lane / 16,
// stored chunk lane % 16 holding global chunk (lane % 16) ^ rm_swz(row).
__device__ inline int rowmajor_off(int b, int lane, int row_bytes) {
  const int row = 4 * b + (lane >> 4);
  const int chunk = (lane & 15) ^ rm_swz(row);
  return row * row_bytes + 16 * chunk;
}

// Lane offsets of the transposing reads that take MFMA operand fragments out
// of a row-major tile (256-byte rows, 16-byte chunks swizzled by rm_swz(row)):
// within each 16-lane group the lanes address a 4-row x 32-byte block, lane
// 4 j + c pointing at 4 columns 4c..4c+3 of row j, so that lane n receives
// column n of the 4 rows. For the 16-row step s (rows 16 s + 4 (lane / 32) +
// 0..3, then + 8: the accumulators' row order) and column block db the two
// reads sit at tile + 4096 s + lo[db] and + hi[db]; row % 16 does not depend
// on s, so neither does the swizzle.
struct TrOffsets {
  int lo[4], hi[4];
  __device__ explicit TrOffsets(int lane) {
    const int rlo = 4 * (lane >> 5) + ((lane >> 2) & 3);
    const int rhi = rlo + 8;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int byte = 64 * db + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
      const int c16 = byte >> 4, within = byte & 15;
      lo[db] = rlo * 256 + 16 * (c16 ^ rm_swz(rlo)) + within;
      hi[db] = rhi * 256 + 16 * (c16 ^ rm_swz(rhi)) + within;
    }
  }
};

__device__ inline bf16x8_t tr_rowmajor(const unsigned char* tile, const TrOffsets& o, int s, int db) {
  const i16x4_t lo = lds_read_tr(tile + 4096 * s + o.lo[db]);
  const i16x4_t hi = lds_read_tr(tile + 4096 * s + o.hi[db]);
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Accumulator registers of a 32x32 block (row 8 (i/4) + 4 half + i%4) packed
// as the operand of the 16-row step s (rows 16 s .. 16 s + 15): registers
// 8 (s & 1) + 0..7 of block s / 2.
__device__ inline bf16x8_t pack_step(const f32x16_t& c, int s) {
  uint4 pk;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int i = 8 * (s & 1) + 2 * jj;
    (&pk.x)[jj] = pack_bf16x2(c[i], c[i + 1]);
  }
  return as_bf16x8(pk);
}

}  // namespace pg_hip
