// Device helpers shared by the matrix-core attention kernels: buffer loads,
// exact fp16 code operands, fp16 hi/lo splits of float32 factors,
// power-of-two prescales, cross-lane reductions on 64-wide waves and the
// split combine.
// Internal header (each kernel translation unit gets its own copy of these
// inline helpers).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned as_u32(float x) { return __builtin_bit_cast(unsigned, x); }
__device__ __forceinline__ float as_f32(unsigned x) { return __builtin_bit_cast(float, x); }

// ---- buffer loads ------------------------------------------------------------
// A buffer descriptor (SGPRs) covers one KV head's array; loads take a 32-bit
// lane offset in a VGPR (and optionally a wave-uniform offset in an SGPR), so
// no 64-bit per-lane address is kept in registers.  A lane offset at or past
// the descriptor's byte count returns zeros without a memory access;
// kNoBlock is such an offset for any array below 2 GiB.
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 raw buffer: 32-bit data, no swizzle
constexpr unsigned kNoBlock = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRawBufferWord3);
}
__device__ __forceinline__ i32x2 buf_b64(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff) {
  return __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ float2 buf_f2(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ f32x4 buf_f4(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// S with max_abs * 2^S in [2^(top-1), 2^top) (0 for a zero maximum), clamped
// so scaled values and inverse factors stay finite and normal in float32.
__device__ __forceinline__ int prescale_exp(float max_abs, int top) {
  if (!(max_abs > 0.0f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(max_abs);
  return min(100, max(-100, top - e));
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return as_f32(static_cast<unsigned>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(as_u32(x)), kCtrl, 0xf, 0xf, true)));
}
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

// Lane ^ 16 and lane ^ 32 exchanges (gfx950 row swaps): returns both halves.
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  a = as_f32(r[0]);
  b = as_f32(r[1]);
}
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  a = as_f32(r[0]);
  b = as_f32(r[1]);
}
// Max / sum over the four 16-lane q-blocks of a wave (lanes n, n^16, n^32, n^48).
__device__ __forceinline__ float qblock_max(float x) {
  float a, b;
  swap16(x, a, b);
  x = fmaxf(a, b);
  swap32(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float qblock_sum(float x) {
  float a, b;
  swap16(x, a, b);
  x = a + b;
  swap32(x, a, b);
  return a + b;
}

// Constants kept in VGPRs: gfx9 VOP3 encodings take no literal operand and
// at most one scalar one, so this lets each nibble extraction be a single
// v_and_or_b32.
struct CodeConsts {
  unsigned lo_mask, hi_mask, magic;
};
__device__ __forceinline__ unsigned in_vgpr(unsigned x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ CodeConsts code_consts() {
  return {in_vgpr(0x000F000Fu), in_vgpr(0x00F000F0u), in_vgpr(0x64006400u)};
}

// Eight code bytes b0..b7 -> fp16 (c - 7) of their low nibbles (lo) and high
// nibbles (hi), in k-slot order (b0, b2, b1, b3, b4, b6, b5, b7).  OR-ing a
// nibble into 0x6400 gives 1024 + c (low) or 1024 + 16c (high, masked in
// place); one packed add, or multiply-add by 1/16, removes the bias exactly.
__device__ __forceinline__ void codes_to_half(i32x2 w, const CodeConsts& k, half8_t& lo,
                                              half8_t& hi) {
  const half2_t bias_lo = {(_Float16)-1031.0f, (_Float16)-1031.0f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t bias_hi = {(_Float16)-71.0f, (_Float16)-71.0f};
  const unsigned src[4] = {static_cast<unsigned>(w.x), static_cast<unsigned>(w.x) >> 8,
                           static_cast<unsigned>(w.y), static_cast<unsigned>(w.y) >> 8};
  u32x4 l, h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned xl = (src[i] & k.lo_mask) | k.magic;
    const unsigned xh = (src[i] & k.hi_mask) | k.magic;
    l[i] = __builtin_bit_cast(unsigned, __builtin_bit_cast(half2_t, xl) + bias_lo);
    h[i] = __builtin_bit_cast(
        unsigned, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, xh), sixteenth, bias_hi));
  }
  lo = __builtin_bit_cast(half8_t, l);
  hi = __builtin_bit_cast(half8_t, h);
}

// 8-bit codes: sixteen code bytes, two rows of 8 (bytes 0..7 and 8..15) ->
// fp16 (c - 127) operands first / second, in the same k-slot order (b0, b2,
// b1, b3, b4, b6, b5, b7) as codes_to_half.  One byte permute places two
// codes under the exponent byte 0x64 (fp16 1024 + c, exact for c < 1024),
// one packed add removes the bias.
struct CodeConsts8 {
  unsigned sel_even, sel_odd, magic;
};
__device__ __forceinline__ CodeConsts8 code_consts8() {
  // v_perm_b32 selectors over {magic (bytes 4..7), word (bytes 0..3)}:
  // (byte 0 | 0x64 << 8 | byte 2 << 16 | 0x64 << 24) and the same for bytes 1, 3.
  return {in_vgpr(0x04020400u), in_vgpr(0x04030401u), in_vgpr(0x64646464u)};
}
__device__ __forceinline__ void codes8_to_half(u32x4 w, const CodeConsts8& k, half8_t& first,
                                               half8_t& second) {
  // (Each value goes through a scalar: __builtin_bit_cast of a vector
  // element compiles to wrong code with this compiler.)
  const half2_t bias = {(_Float16)-1151.0f, (_Float16)-1151.0f};
  const unsigned src[4] = {w.x, w.y, w.z, w.w};
  unsigned out[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned e = __builtin_amdgcn_perm(k.magic, src[i], k.sel_even);
    const unsigned o = __builtin_amdgcn_perm(k.magic, src[i], k.sel_odd);
    out[2 * i] = __builtin_bit_cast(unsigned, __builtin_bit_cast(half2_t, e) + bias);
    out[2 * i + 1] = __builtin_bit_cast(unsigned, __builtin_bit_cast(half2_t, o) + bias);
  }
  const u32x4 a = {out[0], out[1], out[2], out[3]};
  const u32x4 b = {out[4], out[5], out[6], out[7]};
  first = __builtin_bit_cast(half8_t, a);
  second = __builtin_bit_cast(half8_t, b);
}

// Code bytes of one lane's operand pair per format: 8 bytes hold two
// 4-bit rows (low and high nibbles), 16 bytes two 8-bit rows.
template <int kBits>
struct CodeOps;
template <>
struct CodeOps<4> {
  typedef i32x2 words;
  typedef CodeConsts consts;
  static __device__ __forceinline__ consts make() { return code_consts(); }
  static __device__ __forceinline__ words load(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff) {
    return buf_b64(r, voff, soff);
  }
  static __device__ __forceinline__ void to_half(words w, const consts& k, half8_t& a,
                                                 half8_t& b) {
    codes_to_half(w, k, a, b);
  }
};
template <>
struct CodeOps<8> {
  typedef u32x4 words;
  typedef CodeConsts8 consts;
  static __device__ __forceinline__ consts make() { return code_consts8(); }
  static __device__ __forceinline__ words load(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  }
  static __device__ __forceinline__ void to_half(words w, const consts& k, half8_t& a,
                                                 half8_t& b) {
    codes8_to_half(w, k, a, b);
  }
};

// k-slot j of a converted operand holds byte kSlotByte[j] of the 8 read.
__device__ constexpr int kSlotByte[8] = {0, 2, 1, 3, 4, 6, 5, 7};

__device__ __forceinline__ f32x4 mfma(half8_t a, half8_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// x - (float)h for the fp16 h in half `sel` of a packed pair: one
// v_fma_mix_f32 (the fp16 operand is widened inside the instruction).
template <int kSel>
__device__ __forceinline__ float sub_half(float x, unsigned h2) {
  float r;
  if (kSel == 0)
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h2), "v"(x));
  else
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=v"(r) : "v"(h2), "v"(x));
  return r;
}

// fp16 hi/lo split of 8 float32 values, packed in k-slot order: hi rounds
// toward zero, lo is the exact float32 remainder rounded toward zero.
__device__ __forceinline__ void split_hilo(const float x[8], half8_t& hi, half8_t& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned hp = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(x[2 * i], x[2 * i + 1]));
    const float r0 = sub_half<0>(x[2 * i], hp);
    const float r1 = sub_half<1>(x[2 * i + 1], hp);
    h[i] = hp;
    l[i] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(r0, r1));
  }
  hi = __builtin_bit_cast(half8_t, h);
  lo = __builtin_bit_cast(half8_t, l);
}

// ---- phase timestamps (diagnostic build only) -------------------------------
// Built with KVQ_PHASE_TRACE, every wave of a matrix-core attend launch records
// the chip-wide constant 100 MHz clock (s_memrealtime) at fixed points of its
// work into its translation unit's array, one lane per wave, and
// kvq_phase_trace_fetch copies the array out.  In the normal build phase_mark
// compiles to nothing and phase_fetch reports the build as unsupported.
constexpr int kPhaseWaves = 16384;  // waves recorded: the first ones by workgroup, then wave
constexpr int kPhaseMarks = 8;
enum PhaseMark {
  kMarkStart = 0,       // the wave starts
  kMarkQReady = 1,      // its query rows are in registers
  kMarkFirstBlock = 2,  // its first block is ready (4-row kernel)
  kMarkLoopEnd = 3,     // its last block is attended
  kMarkMerged = 4,      // the workgroup's waves are merged
  kMarkAcked = 5,       // the split's partial stores are acknowledged
  kMarkTicket = 6,      // the split took its ticket
  kMarkEnd = 7,         // the wave ends
};
#ifdef KVQ_PHASE_TRACE
__device__ unsigned long long phase_trace[kPhaseWaves * kPhaseMarks];
#endif
__device__ __forceinline__ void phase_mark(int mark) {
#ifdef KVQ_PHASE_TRACE
  const unsigned w = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if ((threadIdx.x & 63) == 0 && w < kPhaseWaves)
    phase_trace[w * kPhaseMarks + mark] = __builtin_amdgcn_s_memrealtime();
#else
  (void)mark;
#endif
}
// Host side: copy up to `bytes` of this translation unit's records.
inline int phase_fetch(void* host, size_t bytes) {
#ifdef KVQ_PHASE_TRACE
  if (bytes > sizeof(phase_trace)) bytes = sizeof(phase_trace);
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(phase_trace), bytes) == hipSuccess ? KVQ_OK
                                                                                : KVQ_ERR_HIP;
#else
  (void)host;
  (void)bytes;
  return KVQ_ERR_UNSUPPORTED;
#endif
}

// ---- issue priority ------------------------------------------------------------
// Priority of this wave among the waves sharing its SIMD before its block i of
// cnt: the share of its blocks still ahead, in the 4 levels of s_setprio.  The
// SIMD then prefers the wave furthest behind, so waves with equal block counts
// finish together instead of the oldest first (which left its workgroup waiting
// at the merge barrier for the youngest).  The caller drops to 0 after its loop.
__device__ __forceinline__ void priority_by_blocks_left(int i, int cnt) {
  switch ((cnt - 1 - i) * 4 / cnt) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}

// ---- split combine -----------------------------------------------------------
// The KV splits of a head merge their partial (m, z, u) rows with the same
// rescale as the blocks ("two stops of the online accumulation" on the
// resource-ledger page: partial statistics compose once brought to one
// reference).  Each workgroup stores its rows with device-scope stores
// (written through to the device coherence point, so no cache flush is
// needed), waits until they are acknowledged, and only then takes a ticket
// from the head's arrival counter; the last to arrive reads every split with
// device-scope loads, writes the output and resets the counter to 0.  (A
// device-scope release/acquire fence would instead write back and invalidate
// the whole L2 of the XCD, once per workgroup.)

// Cache policy of buffer accesses at device scope (gfx9 "sc1"): stores are
// written through to the device coherence point before they are
// acknowledged, loads read it, as for device-scope atomic stores and loads.
constexpr int kCachePolicyDevice = 16;

// Feature of a thread's slot i: runs of kRun consecutive features kStride
// apart, from f0 (consecutive lanes then touch neighbouring words).
template <int kRun, int kStride>
__device__ __forceinline__ int slot_feature(int f0, int i) {
  return f0 + (i / kRun) * kStride + i % kRun;
}

// Buffer descriptor of the u rows of one head in one split.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t split_rows(const AttendProblem& p, int split,
                                                             long long total_rows, long long head) {
  return head_rsrc(p.part_u + (static_cast<long long>(split) * total_rows + head * p.rows) * p.D,
                   static_cast<long long>(p.rows) * p.D * 4);
}

// One workgroup's part of the combine.  Thread: query row r of the head
// (r >= p.rows takes no part), features slot_feature(f0, i), i < kF, its
// merged partial U / M / Z; the thread with f0 == 0 also owns the row's m and
// z.  last: an int of LDS.  Every thread of the workgroup calls this (it
// holds barriers).
// split_store writes one split's partial rows (no wait); split_ticket_merge
// waits for every partial store of the workgroup, takes its ticket for
// `arrivals` splits and, if it is the last, merges the partials in slots
// 0 .. parts - 1.  split_combine is the two for one split (parts = splits).
// A thread's row of the combine: it takes part (mine) when r < p.rows; row
// is the row's index among all B * Hkv * rows query rows.
struct SplitRow {
  bool mine;
  long long total_rows, row;
};
__device__ __forceinline__ SplitRow split_row(const AttendProblem& p, long long head, int r) {
  return {r < p.rows, static_cast<long long>(p.B) * p.Hkv * p.rows, head * p.rows + r};
}

template <int kF, int kRun, int kStride>
__device__ __forceinline__ void split_store(const AttendProblem& p, int split, long long head,
                                            int r, int f0, const float (&U)[kF], float M,
                                            float Z, const SplitRow& sr) {
  const bool mine = sr.mine;
  const long long total_rows = sr.total_rows;
  const long long row = sr.row;
  if (mine) {
    const long long pr = static_cast<long long>(split) * total_rows + row;
    if constexpr (kRun % 4 == 0) {
      // Runs of four features: one 16-byte device-scope store each, so the
      // eight lanes of a row fill whole memory lines.
      const __amdgpu_buffer_rsrc_t rs = split_rows(p, split, total_rows, head);
#pragma unroll
      for (int j = 0; j < kF / 4; ++j) {
        const u32x4 w = {as_u32(U[4 * j]), as_u32(U[4 * j + 1]), as_u32(U[4 * j + 2]),
                         as_u32(U[4 * j + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(
            w, rs, (r * p.D + slot_feature<kRun, kStride>(f0, 4 * j)) * 4, 0, kCachePolicyDevice);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kF; ++i)
        __hip_atomic_store(&p.part_u[pr * p.D + slot_feature<kRun, kStride>(f0, i)], U[i],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (f0 == 0) {
      __hip_atomic_store(&p.part_m[pr], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.part_z[pr], Z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int kF, int kRun, int kStride>
__device__ __forceinline__ void split_ticket_merge(const AttendProblem& p, long long head, int r,
                                                   int f0, int arrivals, int* last,
                                                   const SplitRow& sr, int parts) {
  const bool mine = sr.mine;
  const long long total_rows = sr.total_rows;
  const long long row = sr.row;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the partial stores are acknowledged
  phase_mark(kMarkAcked);
  __syncthreads();
  unsigned* counter = &p.counters[head * kCounterStride];
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, static_cast<unsigned>(arrivals),
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last = ticket_outcome(prev, p.splits, arrivals);
  }
  __syncthreads();
  phase_mark(kMarkTicket);
  if (*last == kTicketWait) return;
  if (*last == kTicketStale) {  // the counter was not zero at the start: make it visible
    if (mine) {
#pragma unroll
      for (int i = 0; i < kF; ++i)  // a quiet NaN, stored as its bit pattern
        reinterpret_cast<unsigned*>(p.out)[row * p.D + slot_feature<kRun, kStride>(f0, i)] =
            0x7fc00000u;
    }
    return;
  }
  if (mine) {
    // Online merge over the partials, four at a time so a batch's loads are
    // in flight together.
    constexpr int kBatch = 4;
    float Mg = -INFINITY, Zg = 0.0f, V[kF];
#pragma unroll
    for (int i = 0; i < kF; ++i) V[i] = 0.0f;
    for (int s0 = 0; s0 < parts; s0 += kBatch) {
      float ms[kBatch], zs[kBatch], us[kBatch][kF];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const long long pr =
            static_cast<long long>(s0 + j < parts ? s0 + j : s0) * total_rows + row;
        ms[j] = __hip_atomic_load(&p.part_m[pr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        zs[j] = __hip_atomic_load(&p.part_z[pr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (kRun % 4 == 0) {
          const __amdgpu_buffer_rsrc_t rs =
              split_rows(p, s0 + j < parts ? s0 + j : s0, total_rows, head);
#pragma unroll
          for (int i4 = 0; i4 < kF / 4; ++i4) {
            const f32x4 x = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           rs, (r * p.D + slot_feature<kRun, kStride>(f0, 4 * i4)) * 4, 0,
                           kCachePolicyDevice));
#pragma unroll
            for (int e = 0; e < 4; ++e) us[j][4 * i4 + e] = x[e];
          }
        } else {
#pragma unroll
          for (int i = 0; i < kF; ++i)
            us[j][i] = __hip_atomic_load(&p.part_u[pr * p.D + slot_feature<kRun, kStride>(f0, i)],
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (s0 + j >= parts) ms[j] = -INFINITY;
      }
      float mb = Mg;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, ms[j]);
      if (mb == -INFINITY) continue;
      const float a = fast_exp2(Mg - mb);  // 0 while nothing is merged yet
      Zg *= a;
#pragma unroll
      for (int i = 0; i < kF; ++i) V[i] *= a;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (ms[j] == -INFINITY) continue;
        const float e = fast_exp2(ms[j] - mb);
        Zg = fmaf(e, zs[j], Zg);
#pragma unroll
        for (int i = 0; i < kF; ++i) V[i] = fmaf(e, us[j][i], V[i]);
      }
      Mg = mb;
    }
#pragma unroll
    for (int i = 0; i < kF; ++i)  // Zg = 0 only for a causal row with no legal key: 0
      p.out[row * p.D + slot_feature<kRun, kStride>(f0, i)] = Zg > 0.0f ? V[i] / Zg : 0.0f;
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int kF, int kRun, int kStride>
__device__ __forceinline__ void split_combine(const AttendProblem& p, int split, long long head,
                                              int r, int f0, const float (&U)[kF], float M,
                                              float Z, int* last) {
  const SplitRow sr = split_row(p, head, r);
  split_store<kF, kRun, kStride>(p, split, head, r, f0, U, M, Z, sr);
  split_ticket_merge<kF, kRun, kStride>(p, head, r, f0, 1, last, sr, p.splits);
}

// Workgroup L of a launch -> (KV head, split).  Workgroups are dealt to the 8
// XCDs round-robin; when the head count is a multiple of 8, the workgroups of
// a head are a multiple of 8 apart, so all of them run on one XCD and their
// partials meet in one L2.  With window parts (the last `win` of a head's
// `per_head` splits), the packed splits of every head come first in the grid
// and the window parts after them: the packed splits then take one compute
// unit each before any second workgroup lands on one, and what shares a
// compute unit is a short window part, not a packed split.
struct WgSlot {
  int head, split;
};
__device__ __forceinline__ WgSlot wg_slot(int L, int heads, int per_head, int win) {
  int count = per_head, base = 0;
  if (win > 0) {
    const int packed = per_head - win;
    if (L < packed * heads) {
      count = packed;
    } else {
      L -= packed * heads;
      count = win;
      base = packed;
    }
  }
  WgSlot s;
  if (heads % 8 == 0) {
    const int slot = L >> 3;
    s.head = (L & 7) + 8 * (slot / count);
    s.split = base + slot % count;
  } else {
    s.head = L / count;
    s.split = base + L % count;
  }
  return s;
}

// ---- recent-token window parts -------------------------------------------------
// A mixed cache ([RL] "prefill and decode": the newest tokens kept in
// float32 beside the packed ones) attended in one launch: the last
// p.win_parts workgroups of each head take the W float32 window tokens
// (positions N .. N + W - 1) in parts of p.win_per_part instead of packed
// blocks, run the same online softmax over them, kWinTile tokens at a time
// through LDS, and join the split combine with their partial (m, z, u) like
// any other split.  The work is small (W is a few dozen tokens) and runs
// beside the packed splits' streaming.
constexpr int kWinD = 128;    // head dimension of the matrix-core kernels
constexpr int kWinTile = 8;   // window tokens per LDS tile

template <int kRowsPad>
struct WinSmem {
  float q[kRowsPad][kWinD + 4];  // q * qscale (padded rows: distinct banks)
  float k[kWinTile][kWinD + 4];
  float v[kWinTile][kWinD];
  float s[kRowsPad][kWinTile + 1];  // scores, then p
  float m[kRowsPad], z[kRowsPad], a[kRowsPad];
};

// Window part `part` of head `head` into this thread's slots: query row r,
// features slot_feature<kRun, kStride>(f0, i), i < kF (the caller's
// split_combine mapping).  Every thread of the workgroup calls it (it holds
// barriers); on return U, M, Z hold the part's u, m, z of row r (m = -inf,
// z = u = 0 for a row with no legal token in the part).
template <int kRowsPad, int kThreadsWG, int kF, int kRun, int kStride>
__device__ __forceinline__ void window_part(const AttendProblem& p, WinSmem<kRowsPad>& ws,
                                            long long head, int part, int r, int f0,
                                            float (&U)[kF], float& M, float& Z) {
  constexpr int kTPD = kThreadsWG / (kRowsPad * kWinTile);  // threads per score dot product
  static_assert(kTPD * kRowsPad * kWinTile == kThreadsWG && (kTPD & (kTPD - 1)) == 0 &&
                    kTPD <= 64, "one power-of-two group of lanes per (row, token) score");
  const int tid = threadIdx.x;
  const int rows = p.rows;
  const int t_lo = part * p.win_per_part;
  const int t_hi = min(p.W, t_lo + p.win_per_part);
  for (int i = tid; i < kRowsPad * kWinD; i += kThreadsWG) {
    const int rr = i / kWinD, d = i % kWinD;
    ws.q[rr][d] = rr < rows ? p.q[(head * rows + rr) * kWinD + d] * p.qscale : 0.0f;
  }
  for (int rr = tid; rr < kRowsPad; rr += kThreadsWG) {
    ws.m[rr] = -INFINITY;
    ws.z[rr] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kF; ++i) U[i] = 0.0f;
  const float* kw = p.k_win + head * p.W * kWinD;
  const float* vw = p.v_win + head * p.W * kWinD;
  // causal limit of a row: its query sits at pos_end - R + r % R
  const int lim0 = p.pos_end - p.R;
  for (int t0 = t_lo; t0 < t_hi; t0 += kWinTile) {
    __syncthreads();  // the previous tile is consumed (first tile: q, m, z are written)
    for (int i = tid; i < kWinTile * kWinD / 4; i += kThreadsWG) {
      const int j = i / (kWinD / 4), d = (i % (kWinD / 4)) * 4;
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, vv = kk;
      if (t0 + j < t_hi) {
        kk = *reinterpret_cast<const f32x4*>(kw + static_cast<long long>(t0 + j) * kWinD + d);
        vv = *reinterpret_cast<const f32x4*>(vw + static_cast<long long>(t0 + j) * kWinD + d);
      }
      *reinterpret_cast<f32x4*>(&ws.k[j][d]) = kk;
      *reinterpret_cast<f32x4*>(&ws.v[j][d]) = vv;
    }
    __syncthreads();
    {  // score of (row rr, token j): kTPD consecutive lanes, then a lane-group sum
      const int dot = tid / kTPD, sub = tid % kTPD;
      const int rr = dot / kWinTile, j = dot % kWinTile;
      float acc = 0.0f;
#pragma unroll 4
      for (int d = sub * 4; d < kWinD; d += 4 * kTPD) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&ws.q[rr][d]);
        const f32x4 b = *reinterpret_cast<const f32x4*>(&ws.k[j][d]);
        acc = fmaf(a[0], b[0], acc);
        acc = fmaf(a[1], b[1], acc);
        acc = fmaf(a[2], b[2], acc);
        acc = fmaf(a[3], b[3], acc);
      }
#pragma unroll
      for (int o = kTPD / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (sub == 0) {
        const int t = t0 + j;
        const bool ok = rr < rows && t < t_hi && (!p.causal || p.N + t <= lim0 + rr % p.R);
        ws.s[rr][j] = ok ? acc : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax of each row over the tile: both z and u move by alpha;
    // a row with no legal token so far keeps m = -inf (exponents against 0)
    for (int rr = tid; rr < kRowsPad; rr += kThreadsWG) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kWinTile; ++j) mx = fmaxf(mx, ws.s[rr][j]);
      const float m_old = ws.m[rr];
      const float m_new = fmaxf(m_old, mx);
      const float m_ref = m_new == -INFINITY ? 0.0f : m_new;
      float sum = 0.0f;
#pragma unroll
      for (int j = 0; j < kWinTile; ++j) {
        const float pj = fast_exp2(ws.s[rr][j] - m_ref);
        ws.s[rr][j] = pj;
        sum += pj;
      }
      const float alpha = fast_exp2(m_old - m_ref);
      ws.z[rr] = fmaf(alpha, ws.z[rr], sum);
      ws.m[rr] = m_new;
      ws.a[rr] = alpha;
    }
    __syncthreads();
    const float alpha = ws.a[r];
#pragma unroll
    for (int i = 0; i < kF; ++i) {
      const int f = slot_feature<kRun, kStride>(f0, i);
      float add = 0.0f;
#pragma unroll
      for (int j = 0; j < kWinTile; ++j) add = fmaf(ws.s[r][j], ws.v[j][f], add);
      U[i] = fmaf(alpha, U[i], add);
    }
  }
  __syncthreads();
  M = ws.m[r];
  Z = ws.z[r];
}

}  // namespace
}  // namespace kvq
