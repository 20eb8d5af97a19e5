// Internal declarations shared by the host layout builder, the C ABI and the
// HIP launchers of libpg.so. Not installed; the public ABI is include/pg.h.
#pragma once

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "pg.h"

// Upload buffer of a layout (pg_pool.cpp): pinned host staging plus a device
// buffer, with one completion event per stream the layout was used on.
constexpr int kSlotEvents = 4;
struct pg_slot {
  int device = -1;
  size_t cap = 0;
  unsigned char* host = nullptr;
  void* dev = nullptr;
  std::mutex mu;                       // guards the event list
  hipEvent_t ev[kSlotEvents] = {};
  hipStream_t stream[kSlotEvents] = {};
  int nev = 0;
  bool overflow = false;               // used on more streams than events
  bool in_use = false;
  bool captured = false;               // used while a stream was being captured:
                                       // a graph may read it at any later time
};
// Takes an idle slot of at least `bytes` on `device` (the current device) or
// makes one. Never waits for the device.
pg_status pg_slot_acquire(int device, size_t bytes, pg_slot** out);
// Records the slot's event for `stream` after work was enqueued there. On a
// stream under graph capture an event record marks nothing on the device, so
// the slot is marked captured instead and is never reused.
void pg_slot_note_use(pg_slot* s, hipStream_t stream);
// Returns the slot; it is reused once its recorded events have completed,
// except a captured slot, which stays reserved until the process ends.
void pg_slot_release(pg_slot* s);

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
  std::vector<int32_t> tok_owner;      // [T] group of a prompt token, response index of a response token
  std::vector<int32_t> suffix_group;   // [N] group of each response
  int32_t max_prefix_len = 0, max_suffix_len = 0;
  int32_t max_group_len = 0;           // longest packed group row (padded-form width)
  std::vector<double> inv_freq;     // [d/2], theta^(-2i/d)
  int32_t max_position = -1;
  int64_t useful_pairs = 0, unpacked_pairs = 0;

  // work list (launch order) and the key spans it references
  int32_t block_tokens = 0, heads_per_item = 0;
  std::vector<pg_work_item> items;
  std::vector<pg_key_span> spans;
  int64_t max_item_cost = 0;
  std::vector<int64_t> xcd_load;   // summed item cost per XCD queue
  std::vector<pg_kv_item> kv_items;   // backward (dK, dV) work list, launch order
  std::vector<pg_dec_item> dec_items;   // decode work list, launch order
  int32_t dec_chunk = 0;                // rows per decode chunk (at most)
  std::vector<int32_t> dec_ref_off;     // [N * Hkv + 1]
  std::vector<int32_t> dec_refs;        // items holding rows of (response, KV head)

  // device copy (one upload slot, filled by pg_layout_upload)
  int device = -1;
  void* dev_buf = nullptr;
  pg_slot* slot = nullptr;
  const int32_t* d_g0 = nullptr;
  const int32_t* d_pe = nullptr;
  const int32_t* d_ss = nullptr;
  const pg_work_item* d_items = nullptr;
  const pg_key_span* d_spans = nullptr;
  const double* d_inv_freq = nullptr;
  const pg_kv_item* d_kv_items = nullptr;
  const int32_t* d_owner = nullptr;          // [T]
  const int32_t* d_group_off = nullptr;      // [G+1]
  const int32_t* d_prefix_lens = nullptr;    // [G]
  const int32_t* d_seg_off = nullptr;        // [G+N+1]
  const int32_t* d_suffix_group = nullptr;   // [N]
  const int32_t* d_suffix_lens = nullptr;    // [N]
  const pg_dec_item* d_dec_items = nullptr;
  const int32_t* d_dec_ref_off = nullptr;    // [N * Hkv + 1]
  const int32_t* d_dec_refs = nullptr;
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
hipError_t pg_launch_pack(const pg_layout& L, const void* prefix, int32_t prefix_pad,
                          const void* suffix, int32_t suffix_pad, void* packed, int64_t row_bytes,
                          hipStream_t stream);
hipError_t pg_launch_unpack(const pg_layout& L, const void* packed, int64_t row_bytes,
                            void* prefix_out, int32_t prefix_pad, void* suffix_out,
                            int32_t suffix_pad, hipStream_t stream);
hipError_t pg_launch_positions_padded(const pg_layout& L, int32_t max_len, int64_t* pos,
                                      uint8_t* mask, hipStream_t stream);
hipError_t pg_launch_pad(const pg_layout& L, const void* packed, int64_t row_bytes, void* padded,
                         int32_t max_len, hipStream_t stream);
hipError_t pg_launch_unpad(const pg_layout& L, const void* padded, int32_t max_len,
                           int64_t row_bytes, void* packed, hipStream_t stream);
hipError_t pg_launch_attn_decode(const pg_layout& L, const void* q, const void* k, const void* v,
                                 const int32_t* cur_lens, void* o, float* lse, void* workspace,
                                 pg_dtype dtype, float softmax_scale, hipStream_t stream);
// Decode step, one workgroup per output row (fp32, or d = 64).
hipError_t pg_launch_decode_rowwise(const pg_layout& L, const void* q, const void* k,
                                   const void* v, const int32_t* cur_lens, void* o, float* lse,
                                   pg_dtype dtype, float softmax_scale, hipStream_t stream);
// Workspace bytes of the decode kernel for layout L (one partial per item).
size_t pg_decode_workspace_bytes(const pg_layout& L);
// Device address of the static decode scratch array (PG_DECODE_SCRATCH_BYTES)
// on `device`, which must be the current device; looked up once per device.
hipError_t pg_decode_scratch(int device, void** ptr);
hipError_t pg_launch_attn_bwd(const pg_layout& L, const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const void* dout, void* dq,
                              void* dk, void* dv, float* delta, float softmax_scale,
                              hipStream_t stream);
// Backward, one wave per query row then one per key row (fp32, or d = 64).
hipError_t pg_launch_bwd_rowwise(const pg_layout& L, const void* q, const void* k, const void* v,
                                 const void* o, const float* lse, const void* dout, void* dq,
                                 void* dk, void* dv, float* delta, pg_dtype dtype,
                                 float softmax_scale, hipStream_t stream);
hipError_t pg_launch_attn_mfma(const pg_layout& L, const void* q, const void* k, const void* v,
                               void* o, float* lse, float softmax_scale, hipStream_t stream);

// Constants the host work list and the MFMA kernel agree on.
constexpr int PG_WAVE_QUERIES = 32;   // query tokens per wave in the MFMA kernel
constexpr int PG_ITEM_WAVES = 8;      // waves per work item (workgroup): two ping-pong groups of 4
constexpr int PG_KEY_TILE = 64;       // keys per LDS tile
constexpr int PG_XCDS = 8;            // XCDs of an MI355X; workgroup p runs on XCD p % 8
constexpr int PG_KV_BLOCK = 128;      // keys per backward dK/dV work item (4 waves x 32)
constexpr int PG_DEC_CHUNK = 512;     // most cache rows per decode work item
constexpr int PG_DEC_LONG_PROMPT = 4096;  // prompts longer than this are chunked by
constexpr int PG_DEC_CHUNK_LONG = 1024;   // up to this many rows per work item
constexpr int PG_DEC_TARGET = 1024;   // decode work items aimed at per step
constexpr int PG_DEC_ROWS = 32;       // most query rows per decode work item (one MFMA column block)
