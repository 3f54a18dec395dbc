// Matrix-core fused attention for the 4- or 8-bit, group-32, D=128 packed
// cache with 5 to 32 query rows per KV head (GQA group x queries), rows
// padded to 16 or 32 so both products fill whole 16x16 matrix-core tiles.
//
// Method: the blocked online softmax of "Block KV decoding: less workspace,
// more time" (huhohoo.com/en/docs/llm/kv-block-decode-cost), section "Do not
// average independently normalized blocks", and of "给长前缀列一张有单位的资源账本"
// (codingai-lec05.pages.dev resource-ledger), section "why FlashAttention need
// not keep the whole heat map": per query row a reference max m, an
// exponential sum z and an unnormalized value sum u relative to 2^m, both
// rescaled by 2^(m_old - m_new) when the reference moves (lazily: only when a
// block's max exceeds it by more than kLazy, so p = 2^(s - m) <= 2^kLazy).
// Waves and KV splits are merged with the same rescale ("two stops of the
// online accumulation" on the same page).
//
// Packed format: the 32-token block byte order of kvq_layout.h, whose K and V
// blocks hand each lane its matrix-core operand bytes at consecutive
// addresses (see the 4-row kernel in kvq_attend_mfma.hip for the byte map).
// Codes become exact fp16 (c - 7) operands (kvq_mfma_common.h).
//
// Math per 32-token block, one wave, row tile t = 0, 1 (rows 16t .. 16t+15):
//   S^T[pair][16t + n] = codes^T (A: 16 token pairs x 32 channels, low and
//     high nibbles as two products) x q~^T (B: 32 channels x 16 rows), with
//     the fp16 hi and lo halves of q~ accumulated into the same tile;
//   u[16t + m][f] += p (A: 16 rows x 32 tokens, fp16 hi and lo) x the value
//     operand of group g (B: 32 tokens x 16 feature pairs).
// The score tile gives lane (n, q) rows 16t + n and tokens 8q .. 8q+7, which
// is exactly the A operand of the value product: no data moves between the
// two products.
//
// q~ = q * qscale * sK[d][G] * kf, formed per block in packed fp16 from the
// hi/lo pairs of q (in registers for the whole kernel, each row prescaled by a
// power of two that puts its largest element in [2^9, 2^10)) and of the
// block's K scales (split once per block, one pair of them per lane, and
// shared through LDS).  kf is a power of two that keeps the block's largest
// K scale in [2^2, 2^5).
//
// The value operand (4-bit codes) carries the V scale: (c - 7) * vh, exact,
// plus (c - 7) * vl, where vh holds the 8 leading bits of the prescaled scale
// sV[token][g] * 2^sv and vl the rest.  Both are shared by the two row tiles,
// so the value product costs three matrix-core products per tile and group
// (ph vh, pl vh, ph vl).  8-bit codes (|c - 127| up to 8 bits) leave no room
// for an exact scale product; there p~ = p * sV * 2^sv is split into fp16
// hi + lo instead.
#include "kvq_internal.h"
#include "kvq_layout.h"
#include "kvq_mfma_common.h"

namespace kvq {
namespace {

constexpr int kW = 4;            // waves per workgroup
constexpr int kT = kW * 64;      // threads per workgroup
constexpr int kR = 32;           // query rows per KV head (padded)
constexpr int kD = 128;
template <int kBits>
constexpr int kBB = 512 * kBits; // K or V code bytes of one 32-token block
template <int kBits>
constexpr int kKStep = 128 * kBits;  // lane code bytes: K k-step stride
template <int kBits>
constexpr int kVStep = 32 * kBits;   //   and V value-group stride
constexpr int kBS = 128;         // K or V scales of one block
constexpr int kQStride = 132;    // LDS row of q: 4 words of padding keep the
                                 // 16 rows read by a quarter-wave on distinct banks
// The reference moves only past m + kLazy (base-2 units), so p <= 2^kLazy.
// 4-bit codes: p goes to the value product as fp16 hi + lo, exact in range up
// to 2^15; 12 makes a move rare even for peaky rows (score spread of several
// units), and each move rescales all of a wave's u.  8-bit codes: p~ = p * sV
// * 2^sv stays below 2^(kLazy + kSvTop) = 2^15.
template <int kBits>
constexpr float kLazy = kBits == 4 ? 12.0f : 6.0f;
constexpr int kSvTop = 9;        // V prescale: max V scale * 2^Sv in [2^8, 2^9),
constexpr int kSvLow = 2;        //   kept while it stays in [2^2, 2^9)
constexpr int kQTop = 10;        // q rows prescaled to max |.| in [2^9, 2^10)
constexpr int kKTop = 5;         // K prescale: max K scale * kf in [2^4, 2^5),
constexpr int kKLow = 2;         //   kept while it stays in [2^2, 2^5)

struct alignas(16) Smem32 {
  union {
    float qs[kR][kQStride];      // q * qscale * 2^Sq(row)
    float wu[2][kR][kD];         // u of two waves at a time, for the merge
    WinSmem<kR> win;             // a recent-token window part
  } u;
  // This block's scale operands, per wave, in the lane order of the products
  // that read them (k-slot order within each 8-wide run):
  //   kops[ks][qb]: fp16 hi (toward zero) and lo of the K scales of channels
  //     32 ks + 8 qb + (0..7), times the block's power-of-two guard kf;
  //   vops[g][qb] (4-bit): fp16 head vh (the 8 leading bits) and remainder vl
  //     of the prescaled V scales of tokens 8 qb + (0..7) in value group g;
  //   svs (8-bit): the prescaled V scales, [group][token].
  u32x4 kops[kW][4][4][2];
  union {
    u32x4 vops[kW][4][4][2];
    float svs[kW][kBS];
  } v;
  float alp[kW][kR];             // rescale factors of a reference move (per wave)
  float qus[kR];                 // 2^-Sq(row)
  float wm[kW][kR];
  float wz[kW][kR];
  int last;
};

template <int kBits>
struct Regs32 {
  typename CodeOps<kBits>::words k[4];  // K codes, k-step 0..3
  typename CodeOps<kBits>::words v[4];  // V codes, value group 0..3
  float2 ks;    // K scales of this lane's k-slot pair (see Lanes32::s_pair)
  float2 vs;    // V scales: 4-bit the same slot pair of one value group,
                // 8-bit scales 2 lane and 2 lane + 1 ([group][token] order)
};

// Buffer descriptors of one KV head's four arrays (kvq_mfma_common.h): the
// block offset rides in an SGPR, the lane offset in a VGPR.
struct Head32 {
  __amdgpu_buffer_rsrc_t kc, ksc, vc, vsc;
};

// Lane (a, qb, j) = (lane / 16, lane / 4 % 4, lane % 4) owns k-slots 2j, 2j + 1
// of run (a, qb): entries 32 a + 8 qb + kSlotByte[2j] and kSlotByte[2j + 1]
// = that + 2 of a block's 128 K scales (channel order) or 4-bit V scales
// ([group][token] order).
struct Lanes32 {
  unsigned k_off, v_off;  // byte offsets of this lane's code bytes in a block
  unsigned s_pair;        // byte offset of its first scale of the slot pair
  unsigned s_off;         // byte offset of scales 2 lane, 2 lane + 1 (8-bit V)
};

__device__ __forceinline__ float buf_f1(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

template <int kBits>
__device__ __forceinline__ void load_scales32(Regs32<kBits>& r, const Head32& h, int blk,
                                              const Lanes32& o) {
  r.ks.x = buf_f1(h.ksc, o.s_pair, blk * kBS * 4);
  r.ks.y = buf_f1(h.ksc, o.s_pair + 8, blk * kBS * 4);
  if constexpr (kBits == 4) {
    r.vs.x = buf_f1(h.vsc, o.s_pair, blk * kBS * 4);
    r.vs.y = buf_f1(h.vsc, o.s_pair + 8, blk * kBS * 4);
  } else {
    r.vs = buf_f2(h.vsc, o.s_off, blk * kBS * 4);
  }
}
template <int kBits>
__device__ __forceinline__ void load_block32(Regs32<kBits>& r, const Head32& h, int blk,
                                             const Lanes32& o) {
  load_scales32(r, h, blk, o);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r.k[i] = CodeOps<kBits>::load(h.kc, o.k_off + i * kKStep<kBits>, blk * kBB<kBits>);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r.v[i] = CodeOps<kBits>::load(h.vc, o.v_off + i * kVStep<kBits>, blk * kBB<kBits>);
}

// Running state of one wave.  Lane (n, q) owns score rows 16t + n (t = 0, 1):
// m[t] is that row's reference max (equal in all its lanes), z[t] the sum of
// p over this lane's tokens 8q .. 8q+7 of every block (summed over the four
// q-blocks at the end).  acc[g][t][e] holds u of rows 16t + 4q + i, features
// 32g + 2n + e, in units of 2^(m + sv).  vscale = 2^sv multiplies the V
// scales parked in LDS; vhi / vlo bound the V scales that keep sv valid.
struct State32 {
  float m[2], z[2];
  f32x4 acc[4][2][2];
  int sv;
  float vscale, vhi, vlo;
  float kf, kun, khi, klo;  // K prescale and the K scales that keep it valid
  bool live;
};

// fp16 hi/lo operands of the 8 products x[j] = a[j] * b[j], j in k-slot
// order: hi = fp16(fp16(a) * fp16(b)) (one packed multiply per pair), lo =
// the residual x - hi, from one fused multiply-add per value rounded once to
// fp16 (v_fma_mixlo_f16 / v_fma_mixhi_f16 widen the fp16 hi internally).
// a, b are float32 with their fp16 (round-toward-zero) pairs a16, b16
// precomputed in the same order.  The eight mix instructions are one asm
// statement with early-clobber outputs (no output shares a register with an
// input), ending with s_nop 1: the compiler's hazard tracking does not see
// inside inline asm, and a matrix-core instruction reading a VGPR that a
// VALU instruction just wrote needs two wait states.
__device__ __forceinline__ void product_hilo(const float a[8], const float b[8],
                                             const half2_t a16[4], const half2_t b16[4],
                                             half8_t& hi, half8_t& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = __builtin_bit_cast(unsigned, a16[i] * b16[i]);
  unsigned l0, l1, l2, l3;
  asm("v_fma_mixlo_f16 %0, %4, %5, -%20 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %6, %7, -%20 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %1, %8, %9, -%21 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %10, %11, -%21 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %2, %12, %13, -%22 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %2, %14, %15, -%22 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %3, %16, %17, -%23 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %3, %18, %19, -%23 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "s_nop 1"
      : "=&v"(l0), "=&v"(l1), "=&v"(l2), "=&v"(l3)
      : "v"(a[0]), "v"(b[0]), "v"(a[1]), "v"(b[1]), "v"(a[2]), "v"(b[2]), "v"(a[3]), "v"(b[3]),
        "v"(a[4]), "v"(b[4]), "v"(a[5]), "v"(b[5]), "v"(a[6]), "v"(b[6]), "v"(a[7]), "v"(b[7]),
        "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]));
  l[0] = l0;
  l[1] = l1;
  l[2] = l2;
  l[3] = l3;
  hi = __builtin_bit_cast(half8_t, h);
  lo = __builtin_bit_cast(half8_t, l);
}

__device__ __forceinline__ half2_t pk16(float x, float y) {
  return __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(x, y));
}

// fp16 lo = a[j] - hi[j] for 8 float32 values a (k-slot order) and their fp16
// hi: one v_fma_mixlo_f16 / v_fma_mixhi_f16 per value (the fp16 hi widened
// inside the instruction, the difference rounded once), with the same
// early-clobber outputs and closing s_nop 1 as product_hilo.
__device__ __forceinline__ half8_t residual_lo(const float a[8], half8_t hi) {
  const u32x4 h = __builtin_bit_cast(u32x4, hi);
  unsigned l0, l1, l2, l3;
  asm("v_fma_mixlo_f16 %0, %4, 1.0, -%12 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %5, 1.0, -%12 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %1, %6, 1.0, -%13 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %7, 1.0, -%13 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %2, %8, 1.0, -%14 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %2, %9, 1.0, -%14 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %3, %10, 1.0, -%15 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %3, %11, 1.0, -%15 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "s_nop 1"
      : "=&v"(l0), "=&v"(l1), "=&v"(l2), "=&v"(l3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]));
  const u32x4 l = {l0, l1, l2, l3};
  return __builtin_bit_cast(half8_t, l);
}

// q~ = q * s as fp16 hi + lo from the fp16 hi/lo pairs of q (qh, ql) and of
// the K scales (sh, sl), all packed fp16 arithmetic: hi = qh * sh rounded to
// nearest, r = qh * sh - hi (exact: the residual of a product of two fp16
// values fits in fp16 outside the subnormal range), lo = (ql * sh + r) +
// qh * sl, each fused multiply-add rounded once.  ql * sl (2^-22 of q~) is
// dropped.
__device__ __forceinline__ void scaled_q(half8_t qh, half8_t ql, half8_t sh, half8_t sl,
                                         half8_t& hi, half8_t& lo) {
  hi = qh * sh;
  const half8_t r = __builtin_elementwise_fma(qh, sh, -hi);
  lo = __builtin_elementwise_fma(qh, sl, __builtin_elementwise_fma(ql, sh, r));
}

// kMasked: mask tokens >= t_end; kCausal (implies kMasked): also mask, for
// score row 16t + n, the tokens after its query's position lim[t], and keep
// rows that have seen no legal key at m = -inf (exponents then taken
// against 0, so (-inf) - (-inf) is never formed).
template <int kBits, int kTiles, bool kMasked, bool kCausal>
__device__ __forceinline__ void attend_block32(Smem32& sm, Regs32<kBits>& br, int tok0, int t_end,
                                               const typename CodeOps<kBits>::consts& cc,
                                               State32& st,
                                               const Head32& h, int next, const Lanes32& lo,
                                               const float us_row[2], const half8_t (&qh)[2][4],
                                               const half8_t (&ql)[2][4], const int (&lim)[2]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;

  // ---- block set-up: scale guards, then this block's scales into LDS ------
  const float lks = fmaxf(br.ks.x, br.ks.y);
  const float lvs = fmaxf(br.vs.x, br.vs.y);
  // K prescale kf = 2^e (scores scaled back by kun = 2^-e): set so the
  // block's largest K scale lands in [2^(kKTop-1), 2^kKTop), kept while it
  // stays in [2^kKLow, 2^kKTop).  The top keeps q~ < 2^15 (q rows below
  // 2^10); the bottom keeps the fp16 lo of scales within 2^4 of the
  // largest out of the subnormal range.
  if (!st.live || __builtin_amdgcn_ballot_w64(!(lks < st.khi)) != 0 ||
      __builtin_amdgcn_ballot_w64(lks >= st.klo) == 0) {
    float mx = fmaxf(lks, dpp<kRowRor1>(lks));
    mx = fmaxf(mx, dpp<kRowRor2>(mx));
    mx = fmaxf(mx, dpp<kRowRor4>(mx));
    mx = qblock_max(fmaxf(mx, dpp<kRowRor8>(mx)));
    const int e = prescale_exp(mx, kKTop);
    st.kf = __builtin_ldexpf(1.0f, e);
    st.kun = __builtin_ldexpf(1.0f, -e);
    st.khi = __builtin_ldexpf(1.0f, kKTop - e);
    st.klo = __builtin_ldexpf(1.0f, kKLow - e);
  }
  const float kf = st.kf, kun = st.kun;
  // V prescale 2^sv: set so the largest V scale lands in [2^8, 2^9), moved
  // only when the block's largest V scale leaves [2^kSvLow, 2^kSvTop) after
  // scaling (u is rescaled by the change; z does not carry it).
  if (!st.live || __builtin_amdgcn_ballot_w64(!(lvs < st.vhi)) != 0 ||
      __builtin_amdgcn_ballot_w64(lvs >= st.vlo) == 0) {
    float vmx = fmaxf(lvs, dpp<kRowRor1>(lvs));
    vmx = fmaxf(vmx, dpp<kRowRor2>(vmx));
    vmx = fmaxf(vmx, dpp<kRowRor4>(vmx));
    vmx = qblock_max(fmaxf(vmx, dpp<kRowRor8>(vmx)));
    const int sv_new = prescale_exp(vmx, kSvTop);
    if (st.live) {
      const float f = __builtin_ldexpf(1.0f, sv_new - st.sv);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          st.acc[g][t][0] *= f;
          st.acc[g][t][1] *= f;
        }
    }
    st.sv = sv_new;
    st.vscale = __builtin_ldexpf(1.0f, sv_new);
    st.vhi = __builtin_ldexpf(1.0f, kSvTop - sv_new);
    st.vlo = __builtin_ldexpf(1.0f, kSvLow - sv_new);
  }
  {
    // This lane's k-slot pair of run (a, qb), written as one word per operand.
    const int a = lane >> 4, qb = (lane >> 2) & 3, j = lane & 3;
    const float k0 = br.ks.x * kf, k1 = br.ks.y * kf;
    const unsigned kh = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(k0, k1));
    const unsigned kl = __builtin_bit_cast(
        unsigned, __builtin_amdgcn_cvt_pkrtz(sub_half<0>(k0, kh), sub_half<1>(k1, kh)));
    unsigned* kw = reinterpret_cast<unsigned*>(&sm.kops[wave][a][qb][0]);
    kw[j] = kh;
    kw[4 + j] = kl;
    if constexpr (kBits == 4) {
      // vh keeps the 8 leading bits of the prescaled scale (exact in fp16, and
      // (c - 7) * vh is exact too: |c - 7| has at most 3 significant bits);
      // vl = the exact float32 remainder, rounded toward zero to fp16.
      const float v0 = br.vs.x * st.vscale, v1 = br.vs.y * st.vscale;
      const float h0 = as_f32(as_u32(v0) & 0xFFFF0000u), h1 = as_f32(as_u32(v1) & 0xFFFF0000u);
      unsigned* vw = reinterpret_cast<unsigned*>(&sm.v.vops[wave][a][qb][0]);
      vw[j] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(h0, h1));
      vw[4 + j] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(v0 - h0, v1 - h1));
    } else {
      float2 v2 = br.vs;
      v2.x *= st.vscale;
      v2.y *= st.vscale;
      *reinterpret_cast<float2*>(&sm.v.svs[wave][2 * lane]) = v2;
    }
  }
  load_scales32(br, h, next, lo);  // next block's scales into the same registers
  const float us0 = us_row[0] * kun, us1 = us_row[1] * kun;

  // ---- S^T = codes^T * q~^T, 4 k-steps of 32 channels, two row tiles ------
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 se[2] = {zero4, zero4}, so[2] = {zero4, zero4};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const half8_t sh = __builtin_bit_cast(half8_t, sm.kops[wave][ks][q][0]);
    const half8_t sl = __builtin_bit_cast(half8_t, sm.kops[wave][ks][q][1]);
    half8_t bh[2], bl[2];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) scaled_q(qh[t][ks], ql[t][ks], sh, sl, bh[t], bl[t]);
    half8_t alo, ahi;  // tokens 2n and 2n + 1
    CodeOps<kBits>::to_half(br.k[ks], cc, alo, ahi);
    br.k[ks] = CodeOps<kBits>::load(h.kc, lo.k_off + ks * kKStep<kBits>,
                                    next * kBB<kBits>);  // next block's k-step
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      se[t] = mfma(alo, bh[t], se[t]);
      se[t] = mfma(alo, bl[t], se[t]);
      so[t] = mfma(ahi, bh[t], so[t]);
      so[t] = mfma(ahi, bl[t], so[t]);
    }
  }

  // raw[t][j]: row 16t + n, token 8q + j, in units of 2^Sq(row) (x kf)
  float raw[2][8];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      raw[t][2 * i] = se[t][i];
      raw[t][2 * i + 1] = so[t][i];
    }
    if (kMasked) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (tok0 + 8 * q + j >= t_end || (kCausal && tok0 + 8 * q + j > lim[t]))
          raw[t][j] = -INFINITY;
    }
  }
  const float us[2] = {us0, us1};
  float lmx[2];
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
    lmx[t] = fmaxf(fmaxf(fmaxf(raw[t][0], raw[t][1]), fmaxf(raw[t][2], raw[t][3])),
                   fmaxf(fmaxf(raw[t][4], raw[t][5]), fmaxf(raw[t][6], raw[t][7]))) * us[t];

  // Move the reference of rows that overshoot it by more than kLazy (a
  // wave-uniform decision).
  if (!st.live || __builtin_amdgcn_ballot_w64(lmx[0] > st.m[0] + kLazy<kBits> ||
                                              (kTiles > 1 && lmx[1] > st.m[1] + kLazy<kBits>)) != 0) {
    float alpha[2];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const float mx = qblock_max(lmx[t]);  // row max over the block (finite unless kCausal)
      const float m_new = st.live ? (mx > st.m[t] + kLazy<kBits> ? mx : st.m[t]) : mx;
      alpha[t] = st.live ? fast_exp2(st.m[t] - m_new) : 0.0f;
      if (kCausal && m_new == -INFINITY) alpha[t] = 0.0f;  // still no legal key: z = u = 0
      st.z[t] *= alpha[t];
      st.m[t] = m_new;
    }
    if (st.live) {
      // acc rows 16t + 4q + i take the factor of score row 16t + 4q + i,
      // owned by lanes n = 4q + i: exchange through this wave's LDS slot.
      if (q == 0) {
        sm.alp[wave][n] = alpha[0];
        if (kTiles > 1) sm.alp[wave][16 + n] = alpha[1];
      }
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.alp[wave][16 * t + 4 * q]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          st.acc[g][t][0] *= a;
          st.acc[g][t][1] *= a;
        }
      }
    }
    st.live = true;
  }

  // p = 2^(s - m) <= 2^kLazy<kBits>; z += sum p.  pk holds p in k-slot order.
  float pk[2][8];
  half2_t p16[2][4];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const float shift = kCausal && st.m[t] == -INFINITY ? 0.0f : -st.m[t];
    float pt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pt[j] = fast_exp2(fmaf(raw[t][j], us[t], shift));
    st.z[t] += ((pt[0] + pt[1]) + (pt[2] + pt[3])) + ((pt[4] + pt[5]) + (pt[6] + pt[7]));
#pragma unroll
    for (int j = 0; j < 8; ++j) pk[t][j] = pt[kSlotByte[j]];
#pragma unroll
    for (int i = 0; i < 4; ++i) p16[t][i] = pk16(pk[t][2 * i], pk[t][2 * i + 1]);
  }

  if constexpr (kBits == 4) {
    // ---- u += p x ((c - 7) * (vh + vl)), one value group at a time ---------
    // p = ph + pl (fp16 hi / lo, shared by the four groups), the V side two
    // fp16 operands per group (shared by both row tiles): (c - 7) * vh exact,
    // (c - 7) * vl rounded once; pl * (c - 7) * vl (2^-19 of the term) is
    // dropped.
    half8_t ph[2], pl[2];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const u32x4 w = {__builtin_bit_cast(unsigned, p16[t][0]), __builtin_bit_cast(unsigned, p16[t][1]),
                       __builtin_bit_cast(unsigned, p16[t][2]), __builtin_bit_cast(unsigned, p16[t][3])};
      ph[t] = __builtin_bit_cast(half8_t, w);
      pl[t] = residual_lo(pk[t], ph[t]);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const half8_t vh = __builtin_bit_cast(half8_t, sm.v.vops[wave][g][q][0]);
      const half8_t vl = __builtin_bit_cast(half8_t, sm.v.vops[wave][g][q][1]);
      half8_t ce, co;  // (c - 7) of features 32g + 2n and 32g + 2n + 1
      CodeOps<kBits>::to_half(br.v[g], cc, ce, co);
      br.v[g] = CodeOps<kBits>::load(h.vc, lo.v_off + g * kVStep<kBits>,
                                     next * kBB<kBits>);  // next block's group
      const half8_t e1 = ce * vh, e2 = ce * vl, o1 = co * vh, o2 = co * vl;
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        st.acc[g][t][0] = mfma(ph[t], e1, st.acc[g][t][0]);
        st.acc[g][t][0] = mfma(pl[t], e1, st.acc[g][t][0]);
        st.acc[g][t][0] = mfma(ph[t], e2, st.acc[g][t][0]);
        st.acc[g][t][1] = mfma(ph[t], o1, st.acc[g][t][1]);
        st.acc[g][t][1] = mfma(pl[t], o1, st.acc[g][t][1]);
        st.acc[g][t][1] = mfma(ph[t], o2, st.acc[g][t][1]);
      }
    }
  } else {
    // ---- u += p~ x V codes, p~ = p * sV * 2^sv, one value group at a time -
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 va = *reinterpret_cast<const f32x4*>(&sm.v.svs[wave][g * 32 + q * 8]);
      const f32x4 vb = *reinterpret_cast<const f32x4*>(&sm.v.svs[wave][g * 32 + q * 8 + 4]);
      float sv[8];  // k-slot order
      sv[0] = va[0]; sv[1] = va[2]; sv[2] = va[1]; sv[3] = va[3];
      sv[4] = vb[0]; sv[5] = vb[2]; sv[6] = vb[1]; sv[7] = vb[3];
      half2_t sv16[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sv16[i] = pk16(sv[2 * i], sv[2 * i + 1]);
      half8_t ah[2], al[2];
#pragma unroll
      for (int t = 0; t < kTiles; ++t) product_hilo(pk[t], sv, p16[t], sv16, ah[t], al[t]);
      half8_t be, bo;  // features 32g + 2n and 32g + 2n + 1
      CodeOps<kBits>::to_half(br.v[g], cc, be, bo);
      br.v[g] = CodeOps<kBits>::load(h.vc, lo.v_off + g * kVStep<kBits>,
                                     next * kBB<kBits>);  // next block's group
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        st.acc[g][t][0] = mfma(ah[t], be, st.acc[g][t][0]);
        st.acc[g][t][0] = mfma(al[t], be, st.acc[g][t][0]);
        st.acc[g][t][1] = mfma(ah[t], bo, st.acc[g][t][1]);
        st.acc[g][t][1] = mfma(al[t], bo, st.acc[g][t][1]);
      }
    }
  }
}

// Issue priority of a wave before its block i of cnt, from the blocks still
// ahead, by a ladder that narrows toward the end: level 3 while more than a
// quarter is ahead, then 2, 1 and 0 below a quarter, an eighth and a
// sixteenth.  The two waves sharing a SIMD (one from each of the compute
// unit's two workgroups) start together with equal runs; the older one gets
// the SIMD's issue slots when their levels tie, so the one behind gets them as
// soon as it falls a level back, and near the end, where the levels are a few
// blocks wide, the two finish within a few blocks of each other instead of the
// younger one running its last third alone at one wave's issue rate.
__device__ __forceinline__ void priority_by_blocks_ahead(int i, int cnt) {
  const int r = cnt - 1 - i;
  if (r * 16 < cnt) __builtin_amdgcn_s_setprio(0);
  else if (r * 8 < cnt) __builtin_amdgcn_s_setprio(1);
  else if (r * 4 < cnt) __builtin_amdgcn_s_setprio(2);
  else __builtin_amdgcn_s_setprio(3);
}

// Several splits per workgroup (kMulti; no window parts).  Workgroup g of a
// head takes splits [s0, s1) = [g spw, min(splits, (g + 1) spw)); wave w
// attends splits s0 + w, s0 + w + kW, ... below s1, each one whole: first
// its masked blocks (the block holding token N-1 when N is not a multiple of
// 32, and with the causal rule the blocks holding tokens past N - R: at most
// two, both at the end of the split), then the others in order.  The wave's
// running (m, z, u) goes on from one of its splits to the next (the online
// merge of their partials; a split of earlier tokens gives every row a legal
// key, so a masked block never meets a row that still needs one after an
// unmasked block); the workgroup then merges its waves as for one split and
// stores one partial, in slot g.  The last arriver merges the head's
// ceil(splits / spw) partials: a two-level combine, with a quarter of the
// partial rows of one partial per split or fewer.
struct WaveSplit {
  int t_end;
  bool active;                    // the split holds a token
  int first;                      // attended first (masked if needed)
  int second;                     // a second masked block, or -1
  int loop_begin, loop_end;       // then these, in order (inclusive)
};
template <bool kCausal>
__device__ __forceinline__ WaveSplit wave_split(const AttendProblem& p, int split) {
  WaveSplit s;
  const int t_begin = split * p.tokens_per_split;
  s.t_end = min(p.N, t_begin + p.tokens_per_split);
  s.active = s.t_end > t_begin;
  const int b_begin = t_begin / kBlockTokens;
  const int b_last = (s.t_end - 1) / kBlockTokens;  // valid if active
  // First block holding a masked token: the causal limit of row 0 (the
  // lowest) is pos_end - R; without the rule only the ragged last block.
  const int b_ragged = (p.N % kBlockTokens) != 0 ? (p.N - 1) / kBlockTokens : INT_MAX;
  const int b_mask = kCausal ? min(b_ragged, (p.pos_end - p.R + 1) / kBlockTokens) : b_ragged;
  const int b_lo = max(b_begin, b_mask);
  const int masked = b_lo <= b_last ? b_last - b_lo + 1 : 0;  // 0, 1 or 2 (pos_end = N)
  s.first = masked > 0 ? b_last : b_begin;
  s.second = kCausal && masked > 1 ? b_last - 1 : -1;
  s.loop_begin = masked > 0 ? b_begin : b_begin + 1;
  s.loop_end = b_last - masked;
  return s;
}

// The wave's splits s, s + kW, ... below s_end into st; br holds split s's
// first block (loaded by the caller when that split is active).
template <int kBits, int kTiles, bool kCausal>
__device__ __forceinline__ void attend_wave_splits(
    const AttendProblem& p, Smem32& sm, Regs32<kBits>& br, const Head32& h, const Lanes32& lo,
    const typename CodeOps<kBits>::consts& cc, State32& st, const float (&us_row)[2],
    const half8_t (&qh)[2][4], const half8_t (&ql)[2][4], const int (&lim)[2], int s,
    int s_end) {
  // The wave's blocks over all its splits, for its issue priority.
  int cnt = 0;
  for (int t = s; t < s_end; t += kW) {
    const WaveSplit w = wave_split<kCausal>(p, t);
    if (w.active) cnt += 1 + (w.second >= 0) + max(0, w.loop_end - w.loop_begin + 1);
  }
  int done = 0;
  WaveSplit sp = wave_split<kCausal>(p, s);
  for (; s < s_end; s += kW) {
    // The block loaded after this split's last one: the wave's next split's first.
    WaveSplit nx = sp;
    int tail_next = -1;
    if (s + kW < s_end) {
      nx = wave_split<kCausal>(p, s + kW);
      if (nx.active) tail_next = nx.first;
    }
    if (sp.active) {
      const bool loop = sp.loop_begin <= sp.loop_end;
      const int after = loop ? sp.loop_begin : (tail_next >= 0 ? tail_next : sp.first);
      priority_by_blocks_ahead(done++, cnt);
      attend_block32<kBits, kTiles, true, kCausal>(
          sm, br, sp.first * kBlockTokens, sp.t_end, cc, st, h,
          sp.second >= 0 ? sp.second : after, lo, us_row, qh, ql, lim);
      if (sp.second >= 0) {
        priority_by_blocks_ahead(done++, cnt);
        attend_block32<kBits, kTiles, true, kCausal>(sm, br, sp.second * kBlockTokens, sp.t_end,
                                                     cc, st, h, after, lo, us_row, qh, ql, lim);
      }
      for (int b = sp.loop_begin; b <= sp.loop_end; ++b) {
        priority_by_blocks_ahead(done++, cnt);
        attend_block32<kBits, kTiles, false, false>(
            sm, br, b * kBlockTokens, sp.t_end, cc, st, h,
            b < sp.loop_end ? b + 1 : (tail_next >= 0 ? tail_next : b), lo, us_row, qh, ql,
            lim);
      }
    } else if (tail_next >= 0) {
      load_block32(br, h, tail_next, lo);
    }
    sp = nx;
  }
}

// kTiles: 16-row tiles of query rows (1 for up to 16 rows per KV head, 2
// for up to 32).  kCausal: a causal chunk (row r is query r % R at position pos_end - R +
// r % R).  Only tokens past pos_end - R can be masked; they lie in at most
// two consecutive blocks (R <= 32), which belong to different waves and are
// each the last block of its wave.  So the masked block of a wave is the one
// it attends first, and its loop runs the unmasked path: every row reads
// every token there, which also gives a row still without a legal key its
// first one.
// kWindow: the last p.win_parts workgroups of each head attend recent-token
// window parts (a separate instantiation, so the plain kernel's block loop is
// compiled without that path).
// kMulti: the workgroup takes p.spw consecutive splits of its head, whole
// splits per wave (attend_wave_splits), stores one partial for all of them
// and takes one ticket for them.
template <int kBits, int kTiles, bool kCausal, bool kWindow, bool kMulti>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attend_mfma_r32_kernel(AttendProblem p) {
  __shared__ Smem32 sm;
  phase_mark(kMarkStart);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;

  // Workgroup -> (KV head, split); with kMulti, `split` is the workgroup's
  // index g in its head, and its run is splits [g spw, (g + 1) spw).  All of
  // a head's workgroups on one XCD when the head count allows (workgroups are
  // dealt to the 8 XCDs round-robin).
  const int heads = p.B * p.Hkv;
  const int wph = kMulti ? (p.splits + p.spw - 1) / p.spw : p.splits;  // workgroups per head
  // Window parts stay among their head's splits here: this kernel's grid
  // often needs more than one round of workgroups, and window parts placed
  // after every packed split would wait for the second.
  const WgSlot wslot = wg_slot(blockIdx.x, heads, wph, 0);
  const int head = wslot.head, split = wslot.split;
  const int s_first = kMulti ? split * p.spw : split;
  const int s_end = kMulti ? min(p.splits, s_first + p.spw) : split + 1;
  const long long bh = head;
  const int rows = p.rows;
  const int packed_splits = p.splits - p.win_parts;
  if (kWindow && split >= packed_splits) {  // a window part (the whole workgroup)
    const int r = tid >> 3, f0 = (tid & 7) * 4;
    float U[16], M, Z;
    window_part<kR, kT, 16, 4, 32>(p, sm.u.win, bh, split - packed_splits, r, f0, U, M, Z);
    split_combine<16, 4, 32>(p, split, bh, r, f0, U, M, Z, &sm.last);
    return;
  }
  // Per-head strides follow the layout's capacity; only blocks below N are read.
  const int nblocks = (p.cap + kBlockTokens - 1) / kBlockTokens;
  Head32 h;
  h.kc = head_rsrc(p.k_codes + bh * nblocks * kBB<kBits>,
                   static_cast<long long>(nblocks) * kBB<kBits>);
  h.ksc = head_rsrc(p.k_scales + bh * nblocks * kBS, static_cast<long long>(nblocks) * kBS * 4);
  h.vc = head_rsrc(p.v_codes + bh * nblocks * kBB<kBits>,
                   static_cast<long long>(nblocks) * kBB<kBits>);
  h.vsc = head_rsrc(p.v_scales + bh * nblocks * kBS, static_cast<long long>(nblocks) * kBS * 4);

  const int t_begin = split * p.tokens_per_split;
  const int t_end = min(p.N, t_begin + p.tokens_per_split);
  const int b_begin = t_begin / kBlockTokens;
  const int b_end = t_end > t_begin ? (t_end + kBlockTokens - 1) / kBlockTokens : b_begin;
  const int b_first = b_begin + wave;
  const int b_last = b_first + (b_end - 1 - b_first) / kW * kW;  // valid if b_first < b_end
  // Code bytes of lane (n, q): K channels 32 ks + 8q .. +7 of tokens 2n, 2n + 1;
  // V tokens 8q .. 8q+7 of features 32 g + 2n, +1 (2 * kBits bytes each).
  // Scales: the k-slot pair (2j, 2j + 1) of run (lane / 16, lane / 4 % 4),
  // entries kSlotByte[2j] = (j & 1) + 4 (j >> 1) and that + 2 of the run.
  const int sj = lane & 3;
  const Lanes32 lo = {static_cast<unsigned>(lane * 2 * kBits),
                      static_cast<unsigned>(q * 128 * kBits + n * 2 * kBits),
                      static_cast<unsigned>(4 * (8 * (lane >> 2) + (sj & 1) + 4 * (sj >> 1))),
                      static_cast<unsigned>(lane * 8)};

  // The block holding token N-1 is masked when N is not a multiple of 32;
  // the wave that owns it attends it first.  Its loads go out before the
  // query rows are staged.
  const bool active = b_first < b_end;
  const bool partial = ((p.N % kBlockTokens) != 0 && b_last == (p.N - 1) / kBlockTokens) ||
                       (kCausal && (b_last + 1) * kBlockTokens - 1 > p.pos_end - p.R);
  const int first = partial ? b_last : b_first;
  const int loop_begin = partial ? b_first : b_first + kW;
  const int loop_end = partial ? b_last - kW : b_last;  // inclusive
  Regs32<kBits> br;
  if constexpr (kMulti) {
    if (s_first + wave < s_end) {
      const WaveSplit w0 = wave_split<kCausal>(p, s_first + wave);
      if (w0.active) load_block32(br, h, w0.first, lo);
    }
  } else if (active) {
    load_block32(br, h, first, lo);
  }

  // q * qscale into LDS, each row prescaled by 2^Sq so its largest element
  // lies in [2^9, 2^10): thread -> (row tid >> 3, channels 16 (tid & 7) ..
  // +15).  Rows past `rows` are zero.
  {
    const int r = tid >> 3, c0 = (tid & 7) * 16;
    float v[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    if (r < rows) {
      const float* qrow = p.q + (bh * rows + r) * kD + c0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(qrow + 4 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * i + j] = a[j] * p.qscale;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    const int sq = prescale_exp(amax, kQTop);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = __builtin_ldexpf(v[4 * i + j], sq);
      *reinterpret_cast<f32x4*>(&sm.u.qs[r][c0 + 4 * i]) = a;
    }
    if ((tid & 7) == 0) sm.qus[r] = __builtin_ldexpf(1.0f, -sq);
  }
  __syncthreads();
  const float us_row[2] = {sm.qus[n], kTiles > 1 ? sm.qus[16 + n] : 1.0f};
  // This lane's q values for the whole kernel (rows 16t + n, channels
  // 32 ks + 8q + (0..7), k-slot order) as fp16 hi (toward zero) and lo of the
  // float32 remainder, kept in registers.
  half8_t qh[2][4], ql[2][4];
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float* qrow = &sm.u.qs[16 * t + n][ks * 32 + q * 8];
      const f32x4 qa = *reinterpret_cast<const f32x4*>(qrow);
      const f32x4 qb = *reinterpret_cast<const f32x4*>(qrow + 4);
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = j < 4 ? qa[kSlotByte[j]] : qb[kSlotByte[j] - 4];
      split_hilo(x, qh[t][ks], ql[t][ks]);
    }

  phase_mark(kMarkQReady);
  const typename CodeOps<kBits>::consts cc = CodeOps<kBits>::make();
  State32 st;
  st.m[0] = st.m[1] = -INFINITY;
  st.z[0] = st.z[1] = 0.0f;
  st.sv = 0;
  st.vscale = 1.0f;
  st.vhi = st.vlo = 0.0f;
  st.kf = st.kun = 1.0f;
  st.khi = st.klo = 0.0f;
  st.live = false;
  {
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int t = 0; t < kTiles; ++t) st.acc[g][t][0] = st.acc[g][t][1] = zero4;
  }

  // Causal limit of this lane's score rows 16t + n.
  const int lim[2] = {p.pos_end - p.R + n % p.R, p.pos_end - p.R + (16 + n) % p.R};
  if constexpr (kMulti) {
    attend_wave_splits<kBits, kTiles, kCausal>(p, sm, br, h, lo, cc, st, us_row, qh, ql, lim,
                                      s_first + wave, s_end);
  } else if (active) {
    const int cnt = 1 + (loop_begin <= loop_end ? (loop_end - loop_begin) / kW + 1 : 0);
    priority_by_blocks_ahead(0, cnt);
    attend_block32<kBits, kTiles, true, kCausal>(sm, br, first * kBlockTokens, t_end, cc, st, h,
                                  loop_begin <= loop_end ? loop_begin : first, lo, us_row, qh,
                                  ql, lim);
    for (int b = loop_begin, i = 1; b <= loop_end; b += kW, ++i) {
      priority_by_blocks_ahead(i, cnt);
      attend_block32<kBits, kTiles, false, false>(sm, br, b * kBlockTokens, t_end, cc, st, h,
                                   min(b + kW, loop_end), lo, us_row, qh, ql, lim);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  phase_mark(kMarkLoopEnd);
  st.z[0] = qblock_sum(st.z[0]);
  if (kTiles > 1) st.z[1] = qblock_sum(st.z[1]);

  // ---- merge the waves: two at a time through LDS -------------------------
  // thread -> (row r = tid >> 3, features f0 + 32 i + (0..3), f0 = 4 (tid & 7))
  const int r = tid >> 3;
  const int f0 = (tid & 7) * 4;
  const float fu = __builtin_ldexpf(1.0f, -st.sv);
  __syncthreads();  // every wave is done with q (aliased by wu)
  if (q == 0) {
    sm.wm[wave][n] = st.m[0];
    sm.wm[wave][16 + n] = kTiles > 1 ? st.m[1] : -INFINITY;  // rows 16..31: none with one tile
    sm.wz[wave][n] = st.z[0];
    sm.wz[wave][16 + n] = kTiles > 1 ? st.z[1] : 0.0f;
  }
  float M = -INFINITY, Z = 0.0f;
  float U[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) U[i] = 0.0f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((wave >> 1) == half) {  // waves 2 half, 2 half + 1 park their u
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float2 u2;
            u2.x = st.acc[g][t][0][i] * fu;
            u2.y = st.acc[g][t][1][i] * fu;
            *reinterpret_cast<float2*>(
                &sm.u.wu[wave & 1][16 * t + 4 * q + i][32 * g + 2 * n]) = u2;
          }
    }
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int w = 0; w < kW; ++w) M = fmaxf(M, sm.wm[w][r]);
    }
    if (M != -INFINITY) {
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2) {
        const float mw = sm.wm[2 * half + w2][r];
        if (mw == -INFINITY) continue;
        const float e = fast_exp2(mw - M);
        Z = fmaf(e, sm.wz[2 * half + w2][r], Z);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.u.wu[w2][r][f0 + 32 * i]);
#pragma unroll
          for (int j = 0; j < 4; ++j) U[4 * i + j] = fmaf(e, a[j], U[4 * i + j]);
        }
      }
    }
    if (half == 0) __syncthreads();  // the first pair is read before the second overwrites it
  }
  phase_mark(kMarkMerged);
  const long long row0 = bh * rows;
  if (p.splits == 1) {
    if (r < rows) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = Z > 0.0f ? U[4 * i + j] / Z : 0.0f;  // Z = 0: no key
        *reinterpret_cast<f32x4*>(&p.out[(row0 + r) * kD + f0 + 32 * i]) = o;
      }
    }
    phase_mark(kMarkEnd);
    return;
  }

  if constexpr (kMulti) {  // slot `split` (the workgroup's index in its head)
    const SplitRow sr = split_row(p, bh, r);
    split_store<16, 4, 32>(p, split, bh, r, f0, U, M, Z, sr);
    split_ticket_merge<16, 4, 32>(p, bh, r, f0, s_end - s_first, &sm.last, sr, wph);
  } else {
    split_combine<16, 4, 32>(p, split, bh, r, f0, U, M, Z, &sm.last);
  }
  phase_mark(kMarkEnd);
}

}  // namespace

// Several splits per workgroup in every form but the causal one with 2 tiles
// of 8-bit codes, whose spills would reach the block loop.  The non-causal
// 2-tile 8-bit form spills 16 bytes per lane, saved before the block loops
// and reloaded after them.
template <int kBits, int kTiles, bool kCausal>
constexpr bool kMultiFits = !(kCausal && kTiles == 2 && kBits == 8);

template <int kBits, int kTiles, bool kCausal>
hipError_t launch_r32c(const AttendProblem& p, unsigned grid, hipStream_t stream) {
  if (p.win_parts > 0) {
    hipLaunchKernelGGL((attend_mfma_r32_kernel<kBits, kTiles, kCausal, true, false>), dim3(grid),
                       dim3(kT), 0, stream, p);
  } else if (p.spw > 1) {
    if constexpr (kMultiFits<kBits, kTiles, kCausal>)
      hipLaunchKernelGGL((attend_mfma_r32_kernel<kBits, kTiles, kCausal, false, true>),
                         dim3(grid), dim3(kT), 0, stream, p);
    else
      return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((attend_mfma_r32_kernel<kBits, kTiles, kCausal, false, false>), dim3(grid),
                       dim3(kT), 0, stream, p);
  }
  return hipGetLastError();
}

template <int kBits, int kTiles>
hipError_t launch_r32(const AttendProblem& p, unsigned grid, hipStream_t stream) {
  return p.causal ? launch_r32c<kBits, kTiles, true>(p, grid, stream)
                  : launch_r32c<kBits, kTiles, false>(p, grid, stream);
}

int phase_fetch_r32(void* host, size_t bytes) { return phase_fetch(host, bytes); }

hipError_t launch_attend_mfma32(const AttendProblem& p, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>((p.splits + p.spw - 1) / p.spw) * p.B * p.Hkv;
  // One 16-row tile when the KV head has at most 16 query rows.
  if (p.bits == 8)
    return p.rows <= 16 ? launch_r32<8, 1>(p, grid, stream) : launch_r32<8, 2>(p, grid, stream);
  return p.rows <= 16 ? launch_r32<4, 1>(p, grid, stream) : launch_r32<4, 2>(p, grid, stream);
}

}  // namespace kvq
