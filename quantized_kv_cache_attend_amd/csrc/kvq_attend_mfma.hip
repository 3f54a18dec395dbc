// Matrix-core fused attention for the 4- or 8-bit, group-32, D=128 packed
// cache with at most 4 query rows per KV head (GQA group x queries <= 4).
//
// Method: the blocked online softmax of "Block KV decoding: less workspace,
// more time" (huhohoo.com/en/docs/llm/kv-block-decode-cost), section "Do not
// average independently normalized blocks", and of "给长前缀列一张有单位的资源账本"
// (codingai-lec05.pages.dev resource-ledger), section "why FlashAttention need
// not keep the whole heat map": per query row a reference max m, an
// exponential sum z and an unnormalized value sum u, both sums relative to
// 2^m and rescaled by 2^(m_old - m_new) whenever the reference moves.
// Scores are in base-2 units (q carries sm_scale * log2 e).  Waves and KV
// splits are merged with the same rescale ("two stops of the online
// accumulation" on the same page: partial statistics are composable).
//
// Lazy reference.  The reference moves only when a block's max exceeds it by
// more than kLazy (2^kLazy bounds every p = 2^(s - m) in between); the pages'
// recurrence moves it on every increase.  Both give the same u / z up to
// rounding (the rescale is exact algebra), and this one skips most rescales.
//
// Packed format ("KV分组打包：4-bit到底省了多少？", huhohoo.com/docs/llm/kv-packed-groups,
// "what a byte holds"), in the 32-token block byte order of kvq_layout.h,
// which puts each lane's matrix-core operand bytes at consecutive addresses:
//   K block (2 KB): lane l = 16 q + n reads 8 bytes at ks*512 + 8 l =
//     channels ks*32 + 8q + (0..7) of token pair n (tokens 2n low nibble,
//     2n+1 high nibble), k-step ks = 0..3;
//   V block (2 KB): lane (n, q) reads 8 bytes at q*512 + g*128 + 8n =
//     tokens 8q + (0..7) of byte column 16g + n (features 32g + 2n, +1);
//   8-bit codes (4 KB blocks): the same lane reads 16 bytes at twice those
//     offsets, the same two rows one byte per code (the first 8 bytes the
//     row of the low nibble above, the next 8 the other);
//   K scales of the block's group: 128 floats, channel order;
//   V scales of the block: [value group][32 tokens].
// Streaming: each wave owns the blocks w, w + kWaves, ... of its split and
// keeps kDepth of them in flight in its own LDS slots: the four parts of a
// block (K codes, V codes, K scales, V scales) are copied from HBM straight
// into LDS by buffer loads with the LDS-destination form and the nontemporal
// cache policy (no VGPRs held while the load is in flight).  When a block's
// loads have landed (vmcnt), every lane reads its operand bytes from the slot
// (contiguous, conflict-free 8- or 16-byte LDS reads in matrix-core operand
// order), and the slot is refilled with the block kDepth ahead before the
// block's math starts.  No barrier is needed before the final merge.
//
// Exact code operands.  Each stored nibble c is turned into the fp16 value
// c - 7 exactly: OR-ing it into the mantissa of 0x6400 gives 1024 + c (low
// nibble) or 1024 + 16c (high nibble, masked in place), and one packed fp16
// add (or multiply-add by 1/16) removes the bias.  All matrix-core operands
// stay in the fp16 normal range: products with fp16 subnormal operands were
// measured to lose low bits when accumulated onto a larger accumulator.
//
// Float32 factors on fp16 matrix cores.  q~[r][d] = q[r][d] * qscale *
// sK[d][G] (scores) and p~[r][j] = p[r][j] * sV[j][G'] (values) are split
// into fp16 hi + lo (round toward zero, then the remainder), so each product
// carries ~22 significant bits and accumulates in float32.  Powers of two
// keep them in the fp16 normal range and are divided out in float32: each
// query row is prescaled once so its largest |q * qscale| lies in [2^9,
// 2^10), which keeps q~ below 2^15 for K scales below 32 (a block with a
// larger K scale is scaled down first), and the V prescale rides in the
// exponent of p (below).
//
// Math per 32-token block, one wave:
//   S^T[pair][col] = codes^T (A: 16 token pairs x 32 channels per k-step,
//     low and high nibbles as two products) x q~^T (B: 32 channels x 16
//     columns; column n = (hi|lo part n >> 3, query row n & 3));
//   u[4 G' + r][f] += p~_G' (A: 16 rows = 4 value groups x 4 query rows)
//     x V codes (B: 32 tokens x 16 feature pairs).
// The A-row layout 4 G' + r lets every lane form the p~ of one value group
// only; rows whose group differs from the B columns' group are discarded.
#include "kvq_internal.h"
#include "kvq_layout.h"
#include "kvq_mfma_common.h"
#include "kvq_quant.h"


namespace kvq {
namespace {

#ifndef KVQ_MFMA_WAVES
#define KVQ_MFMA_WAVES 8
#endif
#ifndef KVQ_MFMA_DEPTH
#define KVQ_MFMA_DEPTH 1
#endif
constexpr int kWaves = KVQ_MFMA_WAVES;   // waves per workgroup, one KV head split each
constexpr int kDepth = KVQ_MFMA_DEPTH;   // blocks in flight per wave (LDS slots)
constexpr int kThreads = kWaves * 64;
constexpr int kOut = 4 * 128;            // outputs of one KV head: 4 rows x D
constexpr int kSlots = kOut / kThreads > 0 ? kOut / kThreads : 1;  // outputs per thread
constexpr int kD = 128;
// K or V code bytes of one 32-token block (4-bit: 2 KB, 8-bit: 4 KB)
template <int kBits>
constexpr int kBB = 512 * kBits;
constexpr int kBS = 128;            // K or V scales of one block
constexpr float kLazy = 6.0f;       // reference moves only past m + kLazy
// V prescale: max V scale * 2^Sv is set to [2^8, 2^9) and kept while it
// stays in [2^2, 2^9): with p <= 2^kLazy, p~ < 2^15 fits fp16.
constexpr int kSvTop = 9;
constexpr int kSvLow = 2;
constexpr int kQTop = 10;           // q rows prescaled to max |.| in [2^9, 2^10)
constexpr float kSkMax = 32.0f;     // K scales below this need no block rescale

// One LDS slot holds a whole block: K codes, V codes, K scales, V scales.
template <int kBits>
constexpr int kSlotBytes = 2 * kBB<kBits> + 2 * kBS * 4;
// Buffer loads with the LDS destination per block: 1 KB per instruction for
// the codes (64 lanes x 16 bytes), half a wave for each 512-byte scale row.
template <int kBits>
constexpr int kDmaPerBlock = 2 * kBB<kBits> / 1024 + 2;
constexpr int kNontemporal = 2;  // cache policy of the block loads (gfx9 "nt")

// LDS of one workgroup.  The merge area and a window part's tiles reuse the
// ring once every block load has landed (8-bit at 8 waves x 2 slots: exactly
// the 160 KB of a compute unit).
struct MergeSmem {
  float wu[kWaves][4][kD];  // per-wave u for the final merge
  float wm[kWaves][4];
  float wz[kWaves][4];
  int last;
};
// Slots per wave: kDepth, or as many as fit in LDS beside the q~ staging
// (8-bit blocks are 9 KB).
constexpr int kQtBytes = kWaves * 4 * 2 * 4 * 4 * 8 * 2;
template <int kBits>
constexpr int kRing = kDepth < (163840 - kQtBytes) / (kWaves * kSlotBytes<kBits>)
                          ? kDepth
                          : (163840 - kQtBytes) / (kWaves * kSlotBytes<kBits>);
static_assert(kRing<8> >= 1, "an 8-bit block must fit in each wave's LDS");

template <int kBits>
struct alignas(16) Smem {
  union {
    unsigned char ring[kWaves][kRing<kBits>][kSlotBytes<kBits>];  // per wave: blocks in flight
    MergeSmem m;
    WinSmem<4> win;                      // a recent-token window part
  } u;
  _Float16 qt[kWaves][4][2][4][4][8];    // per wave: q~ [kstep][hi|lo][row][kblock][8]
};

// One block's operands, as loaded by one lane.
template <int kBits>
struct BlockRegs {
  typename CodeOps<kBits>::words k[4];  // K codes, k-step 0..3
  typename CodeOps<kBits>::words v[4];  // V codes, feature group 0..3
  f32x4 ks[2];  // K scales of channels d0 .. d0+7 (precompute slot)
  f32x4 vs[2];  // V scales of value group n >> 2, tokens 8q .. 8q+7
};

struct Head {
  __amdgpu_buffer_rsrc_t kc, ksc, vc, vsc;
};

// This lane's byte offsets inside a block (precompute slot d0 = channels
// 32 ((lane >> 2) & 3) + 8 (lane & 3) .. +7 for the K scales).  A lane reads
// 2 * kBits code bytes per k-step (K) or feature group (V): channels
// 32 ks + 8q .. +7 of tokens 2n, 2n + 1, and tokens 8q .. 8q+7 of features
// 32 g + 2n, +1; kKStep and kVStep are the strides between them.
template <int kBits>
constexpr int kKStep = 128 * kBits;
template <int kBits>
constexpr int kVStep = 32 * kBits;
struct Lanes {
  unsigned k, v, ks, vs;
};
template <int kBits>
__device__ __forceinline__ Lanes lane_offsets(int lane) {
  const int n = lane & 15, q = lane >> 4;
  const int d0 = ((lane >> 2) & 3) * 32 + (lane & 3) * 8;
  return {static_cast<unsigned>(lane * 2 * kBits),
          static_cast<unsigned>(q * 128 * kBits + n * 2 * kBits), static_cast<unsigned>(d0 * 4),
          static_cast<unsigned>(((n >> 2) * 32 + q * 8) * 4)};
}

#define KVQ_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Copy block `blk` of a head into an LDS slot (asynchronous; counted by
// vmcnt, kDmaPerBlock<kBits> loads per block).  The scale rows take lanes
// 0..31 (16 bytes each), so each lane's LDS destination is the same whether
// the hardware places data by lane id or by active lane.
// valid == false issues the same loads at an offset past the arrays: they
// return zeros without a memory access (keeping the count of loads in flight
// independent of the path taken).
template <int kBits, int kPolicy = kNontemporal>
__device__ __forceinline__ void dma_block(unsigned char* slot, const Head& h, int blk, int lane,
                                          bool valid = true) {
  const unsigned cb = valid ? static_cast<unsigned>(blk) * kBB<kBits> : kNoBlock;
#pragma unroll
  for (int c = 0; c < kBB<kBits> / 1024; ++c) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(h.kc, KVQ_LDS(slot + c * 1024), 16,
                                             cb + c * 1024 + lane * 16, 0, 0, kPolicy);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(h.vc, KVQ_LDS(slot + kBB<kBits> + c * 1024), 16,
                                             cb + c * 1024 + lane * 16, 0, 0, kPolicy);
  }
  if (lane < 32) {
    const unsigned sb = (valid ? static_cast<unsigned>(blk) * kBS * 4 : kNoBlock) + lane * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(h.ksc, KVQ_LDS(slot + 2 * kBB<kBits>), 16, sb, 0, 0,
                                             kPolicy);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(h.vsc, KVQ_LDS(slot + 2 * kBB<kBits> + kBS * 4), 16,
                                             sb, 0, 0, kPolicy);
  }
}

// ---- one-token append in the same launch (decode step) ----------------------
// Workgroup `head` of the grid's front appends token tn = p.N - 1 of that KV
// head with the bytes kvq_append writes for one token ("KV分组打包", "what a
// byte holds"; the cache after n tokens is the pack of those n tokens): the
// open K group (tokens g0 = tn - tn % 32 .. tn of every channel, the earlier
// ones from k_tail) is requantized with its new scale, the token's V row is
// quantized per 32-feature group, and the token joins k_tail unless it
// completes its group.  Every cache store uses the device cache policy
// (written through to the device coherence point); once they are
// acknowledged the head's append flag is raised.  The wave that attends the
// token's block waits for the flag and then loads the block with the same
// policy, so it reads these bytes whichever XCD either workgroup runs on.
constexpr int kCoherent = kNontemporal | kCachePolicyDevice;
constexpr int kAppendSpins = 1 << 16;  // bound on the flag wait (~tens of ms)

template <int kBits>
__device__ void append_token(const AttendProblem& p, int head, float* amax_lds) {
  constexpr int kStep = kBits == 4 ? 2 : 1;  // codes per byte
  constexpr unsigned kZero = Codec<kBits>::kQmaxInt;
  static_assert(kThreads == 4 * kD, "thread (channel d, quarter) of the open K group");
  const Layout L = make_layout(p.cap, kD, kBits, kBlockTokens);
  const int tid = threadIdx.x;
  const long long bh = head;
  const int tn = p.N - 1;
  const int g0 = tn - tn % kBlockTokens;
  // K: thread (d, part) holds tokens g0 + 8 part .. +7 of channel d.
  const int d = tid % kD, part = tid / kD;
  float x[8];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = g0 + 8 * part + j;
    x[j] = t < tn ? p.k_tail[(bh * kBlockTokens + (t - g0)) * kD + d]
                  : (t == tn ? p.k_new[bh * kD + d] : 0.0f);
    amax = fmaxf(amax, fabsf(x[j]));
  }
  amax_lds[part * kD + d] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(amax_lds[d], amax_lds[kD + d]), fmaxf(amax_lds[2 * kD + d], amax_lds[3 * kD + d]));
  const float s = group_scale<kBits>(amax);
  const __amdgpu_buffer_rsrc_t kc =
      head_rsrc(p.k_codes_w + bh * k_code_bytes_per_head(L), k_code_bytes_per_head(L));
#pragma unroll
  for (int j = 0; j < 8; j += kStep) {
    const int t = g0 + 8 * part + j;
    unsigned byte = t <= tn ? stored_code<kBits>(x[j], s) : kZero;
    if (kBits == 4) byte |= (t + 1 <= tn ? stored_code<kBits>(x[j + 1], s) : kZero) << 4;
    __builtin_amdgcn_raw_buffer_store_b8(static_cast<unsigned char>(byte), kc,
                                         static_cast<int>(k_code_byte(L, t, d)), 0,
                                         kCachePolicyDevice);
  }
  if (part == 0)
    __hip_atomic_store(&p.k_scales_w[bh * k_scales_per_head(L) + k_scale_index(L, g0, d)], s,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // The tail is read only by later calls (ordered by the kernel boundary).
  if (part == (tn - g0) / 8 && (tn + 1) % kBlockTokens != 0)
    p.k_tail[(bh * kBlockTokens + tn % kBlockTokens) * kD + d] = x[(tn - g0) % 8];
  // V: thread f0 = kStep * tid of the token's row; 32 / kStep lanes per group.
  if (tid < kD / kStep) {
    const int f0 = kStep * tid;
    const float v0 = p.v_new[bh * kD + f0];
    const float v1 = kStep == 2 ? p.v_new[bh * kD + f0 + 1] : 0.0f;
    float va = fabsf(v0);
    if (kBits == 4) va = fmaxf(va, fabsf(v1));
#pragma unroll
    for (int o = kBlockTokens / kStep / 2; o > 0; o >>= 1) va = fmaxf(va, __shfl_xor(va, o, 64));
    const float sv = group_scale<kBits>(va);
    unsigned byte = stored_code<kBits>(v0, sv);
    if (kBits == 4) byte |= stored_code<kBits>(v1, sv) << 4;
    const __amdgpu_buffer_rsrc_t vc =
        head_rsrc(p.v_codes_w + bh * v_code_bytes_per_head(L), v_code_bytes_per_head(L));
    __builtin_amdgcn_raw_buffer_store_b8(static_cast<unsigned char>(byte), vc,
                                         static_cast<int>(v_code_byte(L, tn, f0)), 0,
                                         kCachePolicyDevice);
    if (f0 % kBlockTokens == 0)
      __hip_atomic_store(&p.v_scales_w[bh * v_scales_per_head(L) + v_scale_index(L, tn, f0)], sv,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores are acknowledged
  __syncthreads();
  if (tid == 0)
    __hip_atomic_store(&p.counters[bh * kCounterStride + kAppendFlag], 1u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// The wave attending the appended token's block: wait (bounded) for the
// head's append flag, then reset it for the next call.  false: it never came.
__device__ __forceinline__ bool wait_append(const AttendProblem& p, int head) {
  unsigned* flag = &p.counters[static_cast<long long>(head) * kCounterStride + kAppendFlag];
  bool up = false;
  for (int spin = 0; spin < kAppendSpins && !up; ++spin) {
    up = __builtin_amdgcn_readfirstlane(
             __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0;
    if (!up) __builtin_amdgcn_s_sleep(2);
  }
  if (up && (threadIdx.x & 63) == 0)
    __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return up;
}

// Wait until at most `pending` blocks' loads (issued after the one needed
// now) are still in flight.
template <int kBits>
__device__ __forceinline__ void wait_blocks(int pending) {
  constexpr int n = kDmaPerBlock<kBits>;
  // s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt at their maxima
#define KVQ_VMCNT(x) (((x) & 15) | (((x) >> 4) << 14) | 0x0F70)
  if (pending <= 0) __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(0));
  else if (pending == 1) __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(n));
  else if (pending == 2) __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(2 * n));
  else __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(3 * n));
#undef KVQ_VMCNT
}

// This lane's operands of the block in `slot`.
template <int kBits>
__device__ __forceinline__ void read_block(BlockRegs<kBits>& r, const unsigned char* slot,
                                           const Lanes& o) {
  typedef typename CodeOps<kBits>::words W;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.k[i] = *reinterpret_cast<const W*>(slot + o.k + i * kKStep<kBits>);
    r.v[i] = *reinterpret_cast<const W*>(slot + kBB<kBits> + o.v + i * kVStep<kBits>);
  }
  const unsigned char* sc = slot + 2 * kBB<kBits>;
  r.ks[0] = *reinterpret_cast<const f32x4*>(sc + o.ks);
  r.ks[1] = *reinterpret_cast<const f32x4*>(sc + o.ks + 16);
  r.vs[0] = *reinterpret_cast<const f32x4*>(sc + kBS * 4 + o.vs);
  r.vs[1] = *reinterpret_cast<const f32x4*>(sc + kBS * 4 + o.vs + 16);
}

// Running state of one wave.  Lane (n, q) tracks query row n & 3: m is the
// row's reference max (the same in all its lanes), z the sum of p over this
// lane's tokens (8q .. 8q+7 of each block; summed over the q-blocks at the
// end).  acc[g][e] holds the value sums of feature group g, even (e = 0) or
// odd (e = 1) features, rows 4q + i = (value group q, query row i), in
// units of 2^(m + sv).  vhi / vlo are the V-scale bounds 2^(kSvTop - sv)
// and 2^(kSvLow - sv) that keep the current sv valid.
struct WaveState {
  float m, z;
  f32x4 acc[4][2];
  int sv;
  float vhi, vlo;
  bool live;  // a block has been folded in
};

// Attend one 32-token block (tokens tok0 .. tok0+31, those >= t_end masked
// out) whose operands are in br.
// qv: this lane's prescaled q values (precompute slot, channel order);
// us_row: 2^-Sq of score row n & 3.  kCausal: also mask the tokens after
// lim, the position of score row n & 3's query; a row that has seen no
// legal key keeps m = -inf and its exponents are taken against 0, so
// (-inf) - (-inf) is never formed.
template <int kBits, bool kCausal>
__device__ __forceinline__ void attend_block(Smem<kBits>& sm, const BlockRegs<kBits>& br,
                                             int tok0, int t_end,
                                             const typename CodeOps<kBits>::consts& cc,
                                             WaveState& ws, const float (&qv)[8], float us_row,
                                             int lim, int lim_lo) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;

  // q~ = q' * sK of this block's K group: lane (rq, ksq, kbq) = (lane >> 4,
  // (lane >> 2) & 3, lane & 3) forms channels ksq*32 + kbq*8 .. +7 of row
  // rq and parks hi / lo in this wave's LDS slots in the B-operand order.
  // A block whose K scales reach kSkMax is scaled by 2^-e first (kun = 2^e
  // restores its scores).
  float kun = 1.0f;
  {
    const int rq = lane >> 4, ksq = (lane >> 2) & 3, kbq = lane & 3;
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = qv[i] * br.ks[0][i];
      x[i + 4] = qv[i + 4] * br.ks[1][i];
    }
    const float lks = fmaxf(fmaxf(fmaxf(br.ks[0][0], br.ks[0][1]), fmaxf(br.ks[0][2], br.ks[0][3])),
                            fmaxf(fmaxf(br.ks[1][0], br.ks[1][1]), fmaxf(br.ks[1][2], br.ks[1][3])));
    if (__builtin_amdgcn_ballot_w64(lks >= kSkMax) != 0) {
      float mx = fmaxf(lks, dpp<kRowRor1>(lks));
      mx = fmaxf(mx, dpp<kRowRor2>(mx));
      mx = fmaxf(mx, dpp<kRowRor4>(mx));
      mx = qblock_max(fmaxf(mx, dpp<kRowRor8>(mx)));
      const int e = __builtin_amdgcn_frexp_expf(mx);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_ldexpf(x[i], -e);
      kun = __builtin_ldexpf(1.0f, e);
    }
    float xs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[j] = x[kSlotByte[j]];
    half8_t hi, lo;
    split_hilo(xs, hi, lo);
    *reinterpret_cast<half8_t*>(&sm.qt[wave][ksq][0][rq][kbq][0]) = hi;
    *reinterpret_cast<half8_t*>(&sm.qt[wave][ksq][1][rq][kbq][0]) = lo;
  }

  // S^T = codes^T * q~^T over 4 k-steps of 32 channels.
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 se = zero4, so = zero4;
  const int part = n >> 3, row = n & 3;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    half8_t alo, ahi;  // tokens 2n and 2n + 1
    CodeOps<kBits>::to_half(br.k[ks], cc, alo, ahi);
    const half8_t b = *reinterpret_cast<const half8_t*>(&sm.qt[wave][ks][part][row][q][0]);
    se = mfma(alo, b, se);
    so = mfma(ahi, b, so);
  }
  const float us = us_row * kun;
  // hi + lo columns: token 8q + t in raw[t], in units of us
  float raw[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    raw[2 * i] = se[i] + dpp<kRowRor8>(se[i]);
    raw[2 * i + 1] = so[i] + dpp<kRowRor8>(so[i]);
  }
  // The block holding token t_end - 1, or (kCausal) one holding a token past
  // N - R that some query may not read; wave-uniform.
  if (tok0 + kBlockTokens > t_end || (kCausal && tok0 + kBlockTokens - 1 > lim_lo)) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (tok0 + 8 * q + t >= t_end || (kCausal && tok0 + 8 * q + t > lim)) raw[t] = -INFINITY;
  }
  // this lane's max over its 8 tokens, base-2 units (us > 0 commutes with max)
  const float lmx =
      fmaxf(fmaxf(fmaxf(raw[0], raw[1]), fmaxf(raw[2], raw[3])),
            fmaxf(fmaxf(raw[4], raw[5]), fmaxf(raw[6], raw[7]))) * us;
  // this lane's largest V scale (value group n >> 2, tokens 8q .. 8q+7)
  const float lvs = fmaxf(fmaxf(fmaxf(br.vs[0][0], br.vs[0][1]), fmaxf(br.vs[0][2], br.vs[0][3])),
                          fmaxf(fmaxf(br.vs[1][0], br.vs[1][1]), fmaxf(br.vs[1][2], br.vs[1][3])));

  // Move the reference when any row's block max overshoots it by more than
  // kLazy, the V prescale when the block's largest V scale leaves
  // [2^kSvLow, 2^kSvTop) after scaling; both decisions are wave-uniform.  A
  // block with no token (a ring step past the wave's last block, never the
  // wave's first step) moves neither and adds p = 0.
  const bool empty = tok0 >= t_end;
  const bool move_m =
      !empty && (!ws.live || __builtin_amdgcn_ballot_w64(lmx > ws.m + kLazy) != 0);
  const bool move_sv = !empty && (!ws.live || __builtin_amdgcn_ballot_w64(!(lvs < ws.vhi)) != 0 ||
                                  __builtin_amdgcn_ballot_w64(lvs >= ws.vlo) == 0);
  if (move_m || move_sv) {
    const float mx = qblock_max(lmx);  // row max over the block (finite unless kCausal)
    float vmx = fmaxf(lvs, dpp<kRowRor4>(lvs));
    vmx = qblock_max(fmaxf(vmx, dpp<kRowRor8>(vmx)));  // block max over the wave
    const float m_new = ws.live ? (mx > ws.m + kLazy ? mx : ws.m) : mx;
    const int sv_new = move_sv ? prescale_exp(vmx, kSvTop) : ws.sv;
    if (ws.live) {
      // a row still without a legal key (kCausal) has z = u = 0: factor 0
      const float alpha = kCausal && m_new == -INFINITY ? 0.0f : fast_exp2(ws.m - m_new);
      ws.z *= alpha;
      const float t = __builtin_ldexpf(1.0f, sv_new - ws.sv);
      const float a0 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 0));
      const float a1 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 1));
      const float a2 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 2));
      const float a3 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 3));
      const f32x4 f = {a0 * t, a1 * t, a2 * t, a3 * t};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        ws.acc[g][0] *= f;
        ws.acc[g][1] *= f;
      }
    }
    ws.m = m_new;
    ws.sv = sv_new;
    ws.vhi = __builtin_ldexpf(1.0f, kSvTop - sv_new);
    ws.vlo = __builtin_ldexpf(1.0f, kSvLow - sv_new);
    ws.live = true;
  }

  // pt = 2^(s - m + Sv) (the V prescale rides in the exponent), z += sum p
  const float shift = static_cast<float>(ws.sv) - (kCausal && ws.m == -INFINITY ? 0.0f : ws.m);
  float pt[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) pt[t] = fast_exp2(fmaf(raw[t], us, shift));
  const float psum = ((pt[0] + pt[1]) + (pt[2] + pt[3])) + ((pt[4] + pt[5]) + (pt[6] + pt[7]));
  ws.z = fmaf(psum, __builtin_ldexpf(1.0f, -ws.sv), ws.z);

  // p~ = pt * sV[token][G'] for this lane's value group, in k-slot order
  half8_t ah, al;
  {
    float xt[8], xv[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      xt[t] = pt[t] * br.vs[0][t];
      xt[t + 4] = pt[t + 4] * br.vs[1][t];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = xt[kSlotByte[j]];
    split_hilo(xv, ah, al);
  }

  // u[4G'+r][f] += p~ x V codes, one feature group of 32 at a time
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    half8_t be, bo;  // features 32g + 2n and 32g + 2n + 1
    CodeOps<kBits>::to_half(br.v[g], cc, be, bo);
    ws.acc[g][0] = mfma(ah, be, ws.acc[g][0]);
    ws.acc[g][0] = mfma(al, be, ws.acc[g][0]);
    ws.acc[g][1] = mfma(ah, bo, ws.acc[g][1]);
    ws.acc[g][1] = mfma(al, bo, ws.acc[g][1]);
  }
}

// kCausal: a causal chunk (row r is query r % R at position N - R + r % R).
// kWindow: the last p.win_parts workgroups of each head attend recent-token
// window parts (a separate instantiation, so the plain kernel's block loop
// is compiled without that path).
// kAppend: the launch also appends token N - 1 (the first B * Hkv workgroups,
// append_token; a separate instantiation, so the plain kernel is unchanged).
template <int kBits, bool kCausal, bool kWindow, bool kAppend>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void
attend_mfma_r4_kernel(AttendProblem p) {
  __shared__ Smem<kBits> sm;
  phase_mark(kMarkStart);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;  // MFMA column / A row
  const int q = lane >> 4;  // MFMA k-block / output row quad

  // Workgroup -> (KV head, split): all splits of a head on one XCD, window
  // parts after every packed split (wg_slot).
  const int heads = p.B * p.Hkv;
  if (kAppend && static_cast<int>(blockIdx.x) < heads) {
    append_token<kBits>(p, blockIdx.x, reinterpret_cast<float*>(&sm.u.ring[0][0][0]));
    return;
  }
  const int L = blockIdx.x - (kAppend ? heads : 0);  // a multiple of 8 apart: same XCD order
  const WgSlot ws_slot = wg_slot(L, heads, p.splits, kWindow ? p.win_parts : 0);
  const int head = ws_slot.head, split = ws_slot.split;
  const long long bh = head;
  const int rows = p.rows;
  const int packed_splits = p.splits - p.win_parts;
  if (kWindow && split >= packed_splits) {  // a window part (the whole workgroup)
    const int e0 = tid * kSlots;
    const int r = e0 >> 7, f0 = e0 & 127;
    float U[kSlots], M, Z;
    window_part<4, kThreads, kSlots, kSlots, 0>(p, sm.u.win, bh, split - packed_splits, r, f0, U,
                                                M, Z);
    split_combine<kSlots, kSlots, 0>(p, split, bh, r, f0, U, M, Z, &sm.u.m.last);
    return;
  }
  // Per-head strides follow the layout's capacity; only blocks below N are read.
  const int nblocks = (p.cap + kBlockTokens - 1) / kBlockTokens;
  Head h;
  h.kc = head_rsrc(p.k_codes + bh * nblocks * kBB<kBits>,
                   static_cast<long long>(nblocks) * kBB<kBits>);
  h.ksc = head_rsrc(p.k_scales + bh * nblocks * kBS, static_cast<long long>(nblocks) * kBS * 4);
  h.vc = head_rsrc(p.v_codes + bh * nblocks * kBB<kBits>,
                   static_cast<long long>(nblocks) * kBB<kBits>);
  h.vsc = head_rsrc(p.v_scales + bh * nblocks * kBS, static_cast<long long>(nblocks) * kBS * 4);

  // Blocks of this split: [b_begin, b_end); wave w takes b_begin + w + i kWaves,
  // i = 0 .. cnt - 1.
  const int t_begin = split * p.tokens_per_split;
  const int t_end = min(p.N, t_begin + p.tokens_per_split);
  const int b_begin = t_begin / kBlockTokens;
  const int b_end = t_end > t_begin ? (t_end + kBlockTokens - 1) / kBlockTokens : b_begin;
  const int b_first = b_begin + wave;
  const int cnt = b_first < b_end ? (b_end - 1 - b_first) / kWaves + 1 : 0;  // wave-uniform

  // This lane's query values: row rq = lane >> 4, channels d0 .. d0+7 (its
  // q~ precompute slot).  Loaded first: the block loads queue behind them,
  // and waiting for q does not wait for any block.
  const int rq = lane >> 4;
  const int d0 = ((lane >> 2) & 3) * 32 + (lane & 3) * 8;
  f32x4 qa = {0.f, 0.f, 0.f, 0.f}, qb = qa;
  if (rq < rows) {
    const float* src = p.q + (bh * rows + rq) * kD + d0;
    qa = *reinterpret_cast<const f32x4*>(src);
    qb = *reinterpret_cast<const f32x4*>(src + 4);
  }
  const Lanes lo = lane_offsets<kBits>(lane);
  // The first kDepth blocks of this wave go out at once (slots past the
  // wave's last block take zeros).
  unsigned char* ring = &sm.u.ring[wave][0][0];
  // With kAppend, the block holding the appended token (the last block of
  // the last split) is loaded only after the append's flag, coherently.
  const int b_app = kAppend ? (p.N - 1) / kBlockTokens : -1;
  bool app_ok = true;
#pragma unroll
  for (int j = 0; j < kRing<kBits>; ++j) {
    const int blk = b_first + j * kWaves;
    if (kAppend && j < cnt && blk == b_app) {
      app_ok = wait_append(p, head);
      dma_block<kBits, kCoherent>(ring + j * kSlotBytes<kBits>, h, blk, lane);
    } else {
      dma_block<kBits>(ring + j * kSlotBytes<kBits>, h, blk, lane, j < cnt);
    }
  }

  // q * qscale, prescaled per row by 2^Sq so the row's largest element lies in
  // [2^9, 2^10) (the 16 lanes of a row are one DPP row).
  float qv[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qv[i] = qa[i] * p.qscale;
    qv[i + 4] = qb[i] * p.qscale;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(qv[i]));
  amax = fmaxf(amax, dpp<kRowRor1>(amax));
  amax = fmaxf(amax, dpp<kRowRor2>(amax));
  amax = fmaxf(amax, dpp<kRowRor4>(amax));
  amax = fmaxf(amax, dpp<kRowRor8>(amax));
  const int sq = prescale_exp(amax, kQTop);
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] = __builtin_ldexpf(qv[i], sq);
  // 2^-Sq of score row n & 3 (held by lanes 16 (n & 3) ..)
  const float us_row = __builtin_ldexpf(1.0f, -__shfl(sq, (n & 3) * 16));
  phase_mark(kMarkQReady);

  const typename CodeOps<kBits>::consts cc = CodeOps<kBits>::make();
  WaveState ws;
  ws.m = -INFINITY;
  ws.z = 0.0f;
  ws.sv = 0;
  ws.vhi = ws.vlo = 0.0f;
  ws.live = false;
  {
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g) ws.acc[g][0] = ws.acc[g][1] = zero4;
  }

  // Causal limit of this lane's score row n & 3.
  const int lim = p.pos_end - p.R + (n & 3) % p.R;

  // The ring: block i sits in slot i % kDepth.  Once its loads have landed
  // and its operands are in registers, the slot is refilled with block
  // i + kDepth, which then streams in while block i is attended.
  for (int i = 0; i < cnt; ++i) {
    priority_by_blocks_left(i, cnt);  // waves that share a SIMD finish together
    wait_blocks<kBits>(min(kRing<kBits> - 1, cnt - 1 - i));
    unsigned char* slot = ring + (i % kRing<kBits>) * kSlotBytes<kBits>;
    BlockRegs<kBits> br;
    read_block(br, slot, lo);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slot has been read
    if (i == 0) phase_mark(kMarkFirstBlock);
    if (i + kRing<kBits> < cnt) {
      const int blk = b_first + (i + kRing<kBits>) * kWaves;
      if (kAppend && blk == b_app) {
        app_ok = wait_append(p, head);
        dma_block<kBits, kCoherent>(slot, h, blk, lane);
      } else {
        dma_block<kBits>(slot, h, blk, lane);
      }
    }
    attend_block<kBits, kCausal>(sm, br, (b_first + i * kWaves) * kBlockTokens, t_end, cc, ws, qv,
                                 us_row, lim, p.pos_end - p.R);
  }
  __builtin_amdgcn_s_setprio(0);
  phase_mark(kMarkLoopEnd);
  if (kAppend && !app_ok) {  // the append never signalled: make the head's output NaN
    const f32x4 nan4 = {as_f32(0x7fc00000u), as_f32(0x7fc00000u), as_f32(0x7fc00000u),
                        as_f32(0x7fc00000u)};
#pragma unroll
    for (int g = 0; g < 4; ++g) ws.acc[g][0] = ws.acc[g][1] = nan4;
  }
  // z of each row: sum this lane's share over the four q-blocks
  ws.z = qblock_sum(ws.z);

  // ---- this wave's u: lanes with q == G hold feature group G ----------------
  f32x4 ue = ws.acc[0][0], uo = ws.acc[0][1];
#pragma unroll
  for (int g = 1; g < 4; ++g) {
    if (q == g) {
      ue = ws.acc[g][0];
      uo = ws.acc[g][1];
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no block load still writes this wave's slots
  __syncthreads();  // every wave is done with its ring (aliased by the merge area)
  const float fu = __builtin_ldexpf(1.0f, -ws.sv);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sm.u.m.wu[wave][i][q * 32 + 2 * n] = ue[i] * fu;
    sm.u.m.wu[wave][i][q * 32 + 2 * n + 1] = uo[i] * fu;
  }
  if (lane < 4) {
    sm.u.m.wm[wave][lane] = ws.m;
    sm.u.m.wz[wave][lane] = ws.z;
  }
  __syncthreads();

  // ---- merge the waves: thread -> row r, features f0 .. f0 + kSlots - 1 ----
  const int e0 = tid * kSlots;
  const int r = e0 >> 7, f0 = e0 & 127;
  float M = -INFINITY, Z = 0.0f, U[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) U[j] = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.u.m.wm[w][r]);
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.u.m.wm[w][r];
      if (mw == -INFINITY) continue;
      const float x = fast_exp2(mw - M);
      Z = fmaf(x, sm.u.m.wz[w][r], Z);
#pragma unroll
      for (int j = 0; j < kSlots; ++j) U[j] = fmaf(x, sm.u.m.wu[w][r][f0 + j], U[j]);
    }
  }
  phase_mark(kMarkMerged);
  const long long row0 = bh * rows;
  if (p.splits == 1) {
    if (r < rows) {
#pragma unroll
      for (int j = 0; j < kSlots; ++j)  // Z = 0: a causal row with no legal key
        p.out[(row0 + r) * kD + f0 + j] = Z > 0.0f ? U[j] / Z : 0.0f;
    }
    phase_mark(kMarkEnd);
    return;
  }
  split_combine<kSlots, kSlots, 0>(p, split, bh, r, f0, U, M, Z, &sm.u.m.last);
  phase_mark(kMarkEnd);
}

}  // namespace

int phase_fetch_r4(void* host, size_t bytes) { return phase_fetch(host, bytes); }

int mfma_tokens_per_split(int N, int splits) {
  const int per = (N + splits - 1) / splits;
  return (per + kBlockTokens - 1) / kBlockTokens * kBlockTokens;
}

template <int kBits, bool kWindow>
void launch_r4(const AttendProblem& p, unsigned grid, hipStream_t stream) {
  if (p.causal)
    hipLaunchKernelGGL((attend_mfma_r4_kernel<kBits, true, kWindow, false>), dim3(grid),
                       dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((attend_mfma_r4_kernel<kBits, false, kWindow, false>), dim3(grid),
                       dim3(kThreads), 0, stream, p);
}

hipError_t launch_attend_mfma(const AttendProblem& p, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(p.splits) * p.B * p.Hkv;
  if (p.append) {  // plain (no window, not causal) attend with the append workgroups in front
    const unsigned g = grid + static_cast<unsigned>(p.B) * p.Hkv;
    if (p.bits == 8)
      hipLaunchKernelGGL((attend_mfma_r4_kernel<8, false, false, true>), dim3(g), dim3(kThreads),
                         0, stream, p);
    else
      hipLaunchKernelGGL((attend_mfma_r4_kernel<4, false, false, true>), dim3(g), dim3(kThreads),
                         0, stream, p);
    return hipGetLastError();
  }
  const bool win = p.win_parts > 0;
  if (p.bits == 8)
    win ? launch_r4<8, true>(p, grid, stream) : launch_r4<8, false>(p, grid, stream);
  else
    win ? launch_r4<4, true>(p, grid, stream) : launch_r4<4, false>(p, grid, stream);
  return hipGetLastError();
}

}  // namespace kvq
