// Internal declarations shared by the library's translation units.
// Not part of the public C ABI (that is include/kvq.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kvq {

// log2(e): scores are kept in base-2 units so the kernels can use exp2.
constexpr float kLog2e = 1.4426950408889634f;

// Largest KV-head row count (GQA heads x queries) the kernels support.
constexpr int kMaxRows = 64;

// One attention problem after validation.
struct AttendProblem {
  const float* q;          // [B][Hq][R][D]
  const uint8_t* k_codes;  // packed (or float32 for the float32-cache path)
  const float* k_scales;
  const uint8_t* v_codes;
  const float* v_scales;
  const float* k_f32;      // float32-cache path only
  const float* v_f32;
  float* out;              // [B][Hq][R][D]
  int B, Hq, Hkv, R, N, D;
  int cap;                 // tokens the packed layout is sized for (>= N; N for float32)
  int causal;              // 1: row r is query r % R at position pos_end - R + r % R (R > 1)
  int pos_end;             // position after the last query (N unless a window follows)
  // Recent-token window, float32 k_win / v_win [B*Hkv][W][D].  General
  // kernel: tokens [N - W, N) are read from it instead of the packed cache.
  // Matrix-core kernels (win_parts > 0): the W window tokens follow the N
  // packed ones; the last win_parts of the `splits` workgroups of a head
  // attend win_per_part window tokens each instead of packed blocks.
  const float* k_win;
  const float* v_win;
  int W;
  int win_parts;
  int win_per_part;
  int rows;                // (Hq / Hkv) * R: query rows sharing one KV head
  int bits, group;         // 4/8 and group; bits == 32 marks the float32 cache
  float qscale;            // sm_scale * log2(e)
  int splits;              // >= 1
  int tokens_per_split;    // ceil(N / splits), rounded up to whole 32-token blocks
  int codes_aligned;       // both code arrays 4-byte aligned (word loads of whole blocks)
  // Workspace views (valid when splits > 1).
  float* part_m;           // [splits][B*Hkv*rows]
  float* part_z;           // [splits][B*Hkv*rows]
  float* part_u;           // [splits][B*Hkv*rows][D]
  unsigned* counters;      // [B*Hkv][kCounterStride], one arrival counter per KV head
  // One-token append in the same launch (4-row matrix-core kernel): token
  // N - 1 of every KV head is appended by B * Hkv extra workgroups at the
  // front of the grid, exactly as kvq_append appends one token; the wave that
  // attends the token's block waits for the head's append flag first.
  int append;              // 1: this launch appends token N - 1
  const float* k_new;      // [B*Hkv][D] float32 K and V of the new token
  const float* v_new;
  float* k_tail;           // [B*Hkv][group][D], as kvq_append reads and writes it
  uint8_t* k_codes_w;      // the cache arrays again, written by the append
  float* k_scales_w;
  uint8_t* v_codes_w;
  float* v_scales_w;
  int spw;                 // splits per workgroup (32-row kernel; 1 in every other kernel)
};

// Append flag of a KV head: word 32 of the head's counter slot (its own
// memory line).  The append raises it to 1 once its stores are acknowledged;
// the waiting wave resets it to 0, so every completed call leaves it zero.
constexpr int kAppendFlag = 32;

// Arrival counters sit 256 bytes apart, so the heads' tickets never contend
// for one memory line.
constexpr int kCounterStride = 64;

// What a workgroup's ticket (the counter's value before its increment) says:
// wait (other splits are still running), merge (it is the last of `splits`),
// or stale (the counter was not zero when the call started, so no ticket can
// be trusted: the workspace was not zero-filled as required).  A stale head's
// output is written as NaN by every workgroup that sees it, and its counter
// is left non-zero, so the failure shows in this call and in every later one
// until the workspace is zero-filled again.
// A workgroup that completes `arrivals` splits at once (one fetch-add of
// `arrivals`) is the last when its ticket reaches `splits` exactly.
constexpr int kTicketWait = 0, kTicketMerge = 1, kTicketStale = 2;
__host__ __device__ inline int ticket_outcome(unsigned prev, int splits, int arrivals = 1) {
  const unsigned s = static_cast<unsigned>(splits);
  const unsigned a = static_cast<unsigned>(arrivals);  // 1 <= arrivals <= splits
  return prev == s - a ? kTicketMerge : (prev >= s - a + 1 ? kTicketStale : kTicketWait);
}

// Workspace carving, shared by the sizing call and the launchers.
struct WorkspaceLayout {
  size_t m_off, z_off, u_off, cnt_off, total;
};
WorkspaceLayout workspace_layout(int B, int Hq, int Hkv, int R, int D, int splits);

// Launchers (host functions; return the launch's hipError_t).
hipError_t launch_pack(const float* x, int B, int H, int N, int D, int bits, int group,
                       bool k_style, uint8_t* codes, float* scales, hipStream_t stream);
// Empty-cache state (every code the zero code, every scale 1) and the
// decode-step append of T tokens after the first N of a cache laid out for
// `cap` tokens; k_tail [B*H][group][D] keeps the float32 K of the tokens of
// the open K group.
hipError_t launch_cache_clear(int B, int H, int cap, int D, int bits, int group, uint8_t* k_codes,
                              float* k_scales, uint8_t* v_codes, float* v_scales,
                              hipStream_t stream);
hipError_t launch_append(const float* k_new, const float* v_new, int B, int H, int N, int T,
                         int cap, int D, int bits, int group, uint8_t* k_codes, float* k_scales,
                         uint8_t* v_codes, float* v_scales, float* k_tail, hipStream_t stream);
hipError_t launch_dequant(const uint8_t* codes, const float* scales, int B, int H, int N, int D,
                          int bits, int group, bool k_style, float* out, hipStream_t stream);
hipError_t launch_attend_valu(const AttendProblem& p, hipStream_t stream);
hipError_t launch_attend_mfma(const AttendProblem& p, hipStream_t stream);
// Matrix-core kernels: up to kMfmaMaxRows query rows per KV head (4-row
// kernel) and up to kMfma32MaxRows (32-row kernel); both take splits in
// whole 32-token blocks.
constexpr int kMfmaMaxRows = 4;
constexpr int kMfma32MaxRows = 32;
int mfma_tokens_per_split(int N, int splits);
hipError_t launch_attend_mfma32(const AttendProblem& p, hipStream_t stream);
// Streaming float32 kernel: 4- or 8-bit, power-of-two group in [8, 128],
// D = 128, up to kStreamMaxRows query rows per KV head, no causal rule and no
// float32 window.
constexpr int kStreamMaxRows = 8;
hipError_t launch_attend_stream(const AttendProblem& p, hipStream_t stream);
int stream_waves(int bits, int rows);  // waves per workgroup of that launch
// Phase records of the 4-row / 32-row / streaming kernels (a kvq_status;
// KVQ_ERR_UNSUPPORTED unless built with KVQ_PHASE_TRACE).
int phase_fetch_r4(void* host, size_t bytes);
int phase_fetch_r32(void* host, size_t bytes);
int phase_fetch_stream(void* host, size_t bytes);
hipError_t launch_stream_read(const void* data, long long bytes, unsigned* sink,
                              hipStream_t stream);

}  // namespace kvq
