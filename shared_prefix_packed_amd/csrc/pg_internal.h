// Internal declarations shared by the host layout builder, the C ABI and the
// HIP launchers of libpg.so. Not installed; the public ABI is include/pg.h.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "pg.h"

struct pg_layout {
  // shape
  int32_t G = 0;
  int32_t num_segments = 0;
  int32_t Hq = 0, Hkv = 0, d = 0;
  int64_t T = 0;
  double rope_theta = 0.0;

  // host copies of the inputs and the derived tables
  std::vector<int32_t> prefix_lens, suffix_counts, suffix_lens;
  std::vector<int32_t> group_off;   // [G+1]
  std::vector<int32_t> seg_off;     // [num_segments+1]
  std::vector<int32_t> tok_g0, tok_pe, tok_ss;   // [T]
  std::vector<double> inv_freq;     // [d/2], theta^(-2i/d)
  int32_t max_position = -1;
  int64_t useful_pairs = 0, unpacked_pairs = 0;

  // work list (launch order) and the key spans it references
  int32_t block_tokens = 0, heads_per_item = 0;
  std::vector<pg_work_item> items;
  std::vector<pg_key_span> spans;
  int64_t max_item_cost = 0;
  std::vector<int64_t> xcd_load;   // summed item cost per XCD queue

  // device copy (one allocation, filled by pg_layout_upload)
  int device = -1;
  void* dev_buf = nullptr;
  std::vector<unsigned char> staging;   // host image of dev_buf, kept alive for the async copy
  const int32_t* d_g0 = nullptr;
  const int32_t* d_pe = nullptr;
  const int32_t* d_ss = nullptr;
  const pg_work_item* d_items = nullptr;
  const pg_key_span* d_spans = nullptr;
  const double* d_inv_freq = nullptr;
};

// Host layout builder (pg_layout.cpp). Validates and fills `L`.
pg_status pg_layout_build_host(pg_layout& L, int32_t num_groups, const int32_t* prefix_lens,
                               const int32_t* suffix_counts, const int32_t* suffix_lens,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               double rope_theta);

// Error text of the calling thread (pg_capi.cpp).
pg_status pg_fail(pg_status s, const char* fmt, ...);
void pg_clear_error();

// Kernel launchers (pg_kernels.hip, pg_attn_mfma.hip). Each returns the
// launch status (hipGetLastError after the launch).
hipError_t pg_launch_positions(const pg_layout& L, int64_t* pos, hipStream_t stream);
hipError_t pg_launch_rope(const pg_layout& L, const int64_t* pos, const void* q_in,
                          const void* k_in, void* q_out, void* k_out, pg_dtype dtype,
                          hipStream_t stream);
hipError_t pg_launch_attn_rowwise(const pg_layout& L, const void* q, const void* k,
                                  const void* v, void* o, float* lse, pg_dtype dtype,
                                  float softmax_scale, hipStream_t stream);
hipError_t pg_launch_attn_mfma(const pg_layout& L, const void* q, const void* k, const void* v,
                               void* o, float* lse, float softmax_scale, hipStream_t stream);

// Constants the host work list and the MFMA kernel agree on.
constexpr int PG_WAVE_QUERIES = 32;   // query tokens per wave in the MFMA kernel
constexpr int PG_ITEM_WAVES = 8;      // waves per work item (workgroup): two ping-pong groups of 4
constexpr int PG_KEY_TILE = 64;       // keys per LDS tile
constexpr int PG_XCDS = 8;            // XCDs of an MI355X; workgroup p runs on XCD p % 8
