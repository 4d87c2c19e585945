// Indexer scoring kernel for gfx950:
//   I[t, s] = k_scale[s] * sum_h w'[t, h] * max(0, <q8[t, h, :], k8[s, :]>),  w' = w * q_scale * scale
// for fp8 keys, and with the MXFP4 E8M0 block scales applied inside the MFMA for fp4 keys.
// Folding the positive scales out of the ReLU is exact in real arithmetic
// (max(0, a x) = a max(0, x) for a >= 0).  The contraction over D = 128 runs on
// v_mfma_scale_f32_16x16x128_f8f6f4; the ReLU, head weighting and head sum run
// straight from the accumulators, on an f16 MFMA or on the VALU (P1 section 1: the
// dense indexer scores T rows against the whole prefix; P2 Motivation: fp8 q x fp4 k).
//
// Two forms of the kernel serve one launch, over the same grid; each workgroup
// works in one of them, by its rows' head weights.
//   f16 form (every weight >= 0): the fp8 MFMA runs with an A-scale of 2^-SA, so
//   every possible dot lies in (-1, 1); one clamping conversion to f16 per two
//   values is the ReLU; an f16 MFMA whose A holds each query's weights (hi and lo
//   f16 parts, block-diagonal) sums the heads, one per two fp8 MFMAs.  The terms
//   carry f16 rounding (2^-11 relative), which bounds the score's relative error
//   only when no weight is negative.
//   fp32 form (any other row): ReLU and weighted head sum as an fp32 FMA chain.
//
// Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4, as measured on gfx950:
// lane l holds row (A) / column (B) l % 16; for fp8, byte b of lane group
// g = l / 16 is k = 64 (b / 16) + 16 g + b % 16; for fp4, nibble p (low nibble
// first) of lane group g is k = 32 g + p; lane l's E8M0 scale covers its row /
// column and k block l / 16 (32 consecutive k); the result C[4 (l / 16) + j][l % 16]
// is element j of lane l.  So an MXFP4 key's 32-element scale block is exactly
// one lane's 16 bytes and one lane's scale byte.
//
// Work decomposition.  The 16 A rows of one MFMA are QR query rows x HPT heads
// (QR = 128 / H: HPT = 4 for H = 32, 8 for H = 64), and a wave owns NT = 8
// such tiles: all H heads of its QR query rows, held in registers (64 VGPRs of
// q, 32 of w') for the whole launch.  Lane l then accumulates heads of query
// (4 (l / 16)) / HPT for key l % 16, so the fp32 form's head sum is an in-lane FMA
// chain plus, for H = 64, one v_permlane16_swap add.
//
// Keys stream through LDS in 16 KiB stages (128 fp8 keys or 256 MXFP4 keys),
// triple buffered and written by the memory system directly
// (global_load_lds_dwordx4): stage i + 2 is requested while stage i is scored.
// Each wave waits only for its own requests (s_waitcnt vmcnt with the number of
// memory operations it has issued since, at least) and then meets the others at
// a barrier.  16-byte chunks are XOR-swizzled inside an LDS row so that the 16
// lanes reading one chunk column hit distinct banks.  LDS row p holds key
// 64 (p / 64) + 4 (p % 16) + (p / 16) % 4, so the 16-key group j of a 64-key
// batch gives lane n the key 64 b + 4 n + j: after a batch every lane holds 4
// consecutive keys of its query row (one 16-byte store, one 16-byte k_scale
// read, an in-lane 8-key max).
// Output stores go through a buffer resource; lanes with nothing to store get
// an out-of-range offset, so stores never branch.  MFMA results land in VGPRs
// (VGPR-form MFMA): the fp32 form's epilogue costs 2 VALU ops per (t, h, s) (a
// max and an FMA), the f16 form's half an op plus a quarter of an f16 MFMA.
//
// Grid: (row blocks of RPW rows) x (nsplit key splits), in one of two layouts
// (workgroup b runs on XCD b % 8, round-robin dispatch).  By key split (the
// default): workgroup b takes split b % nsplit, row block b / nsplit; with nsplit
// a multiple of 8 every split's workgroups land on one XCD, so each XCD's L2 only
// ever holds 1/8 of the keys.  By row block, when the rows' windows cover less than
// half of the launch's keys (a per-launch flag computed on the device from the
// windows): row blocks == b (mod 8) run on XCD b % 8 with all their splits, so a
// ragged batch of short requests, whose active items all sit in a few splits,
// still spreads over every XCD.
#include "kernels.h"

#include <algorithm>
#include <atomic>
#include <climits>
#include <type_traits>

namespace idx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Two fp32 values to packed f16, rounded to nearest even, each clamped to [0, 1]: the
// compiler folds the clamp into the conversion's clamp bit (one v_cvt_pk_f16_f32 ... clamp).
// With every score term scaled into [-1, 1] beforehand, this is the ReLU and the f16
// rounding in one VALU operation.
__device__ __forceinline__ uint32_t cvt_relu_f16x2(float lo, float hi) {
  v2h h = __builtin_convertvector((v2f){lo, hi}, v2h);
  h = __builtin_elementwise_min(__builtin_elementwise_max(h, (v2h){0, 0}), (v2h){1, 1});
  return __builtin_bit_cast(uint32_t, h);
}

// ReLU as one integer max: a float with the sign bit set is a negative int32
// and becomes +0, a non-negative float keeps its bits (fmaxf would add a NaN
// canonicalisation, a second VALU op per value).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

typedef __attribute__((address_space(3))) unsigned char lds_u8;
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(const lds_u8 *)p; }

// Memory-to-LDS copies: lane l's 16 (4) bytes at g land at LDS byte lds + 16 l (4 l);
// lds is wave-uniform.  m0 carries the LDS base into the copy.  The compiler reserves
// m0 and never keeps a value of its own there across statements (it is not
// preserved across asm either), and nothing else in these kernels uses it.
__device__ __forceinline__ void lds_copy16(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}
__device__ __forceinline__ void lds_copy4(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory");
}
// Inclusive prefix sum over the 16 lanes of a DPP row, and that row's total.
__device__ __forceinline__ uint32_t row16_scan(uint32_t x, uint32_t &total) {
  // row total by a butterfly (quad swaps, half-row and row mirrors), all on DPP: no LDS
  // instruction, so no wait on the key reads in flight
  uint32_t t = x;
  t += (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
  t += (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0x4E, 0xF, 0xF, false);   // quad [2,3,0,1]
  t += (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0x141, 0xF, 0xF, false);  // row half mirror
  t += (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0x140, 0xF, 0xF, false);  // row mirror
  total = t;
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  return x;
}

// The value is in registers here (a use the compiler cannot move or drop).
__device__ __forceinline__ void in_regs(v8i x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void in_regs(v4i x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void in_regs(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void in_regs(int x) { asm volatile("" ::"v"(x)); }
// Wait until at most N of this wave's memory operations are outstanding (they complete
// in issue order), then meet the workgroup.  The memory clobber keeps LDS reads after it.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

constexpr int OOB = (int)0x80000000;  // buffer offset past any num_records: the store is dropped
constexpr int RSRC3 = 0x00020000;     // raw buffer, 32-bit elements

// Chunk swizzle inside a key row.  fp8 rows hold 8 chunks of 16 bytes; MXFP4 rows 4.
__device__ __forceinline__ int swz8(int n) { return (n & 7) ^ ((n >> 3) & 1); }
__device__ __forceinline__ int swz4(int n) { return ((n >> 1) ^ (n >> 3)) & 3; }

template <int KF, int H, int MODE, int NW, bool F16>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(!F16 && MODE != STORE_DENSE && MODE != STORE_BLOCK ? 2 : 3))) void logits_kernel(LogitsArgs a) {
  constexpr int QR = 128 / H;            // query rows per wave
  constexpr int HPT = 16 / QR;           // heads of one row in a 16-row A tile
  constexpr int NT = H / HPT;            // A tiles per wave (8)
  constexpr int RPW = NW * QR;           // rows per workgroup
  constexpr int KB = KF == 0 ? 128 : 64; // key bytes
  constexpr int TK = KF == 0 ? 128 : 256; // keys per LDS stage (16 KiB either way)
  constexpr int BY_ROW_MIN_TILES = 4;
  constexpr int STAGE = TK * KB;
  constexpr int LPT = STAGE / 16 / (NW * 64);  // 16-byte chunks per thread per stage
  constexpr int ST = MODE == STORE_SLAB ? 0 : TK / 64;  // stores per stage and wave, at least (candidate stores on top)
  static_assert(LPT * NW * 64 * 16 == STAGE, "stage must split evenly over the workgroup");
  static_assert(RPW <= 64 && TK <= NW * 64 && TK % 64 == 0, "layout limits");

  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[3][STAGE];
  __shared__ __attribute__((aligned(256))) uint32_t sbuf[3][TK];
  __shared__ int32_t wg_range[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (keeps buffer resources scalar)
  // work item and part: the first nfull workgroups take item blockIdx.x whole, the rest
  // take part `part` of `nparts` of a later item.  With splits and remainder in whole
  // multiples of 8, a remainder workgroup stays on the XCD of its item's split
  // (workgroup b runs on XCD b % 8, and so do the splits s with s % 8 == b % 8).
  // fp32 form: nothing to do unless an f16-form workgroup of this launch pair found rows
  // with a negative head weight (uniform)
  if (!F16 && *a.neg_seq < a.seq) return;
  if (a.by_row && (*a.by_row & 2u) != 0u) return;   // no window key in the launch (uniform)
  if (a.kshift) {   // the row chunk's launches start at its first window key
    const int sh = *a.kshift;
    a.key_lo = min(a.key_lo + sh, a.L);
    a.key_hi = min(a.key_hi + sh, a.L);
  }
  const int b = blockIdx.x;
  int item = b, part = 0, nparts = 1;
  if (b >= a.nfull) {
    const int t = b - a.nfull;
    nparts = a.parts;
    if ((a.nsplit & 7) == 0 && (a.nfull & 7) == 0) {
      const int i = t >> 3;
      item = a.nfull + (t & 7) + 8 * (i / nparts);
      part = i % nparts;
    } else {
      item = a.nfull + t / nparts;
      part = t % nparts;
    }
  }
  // Items are (row block, key split) pairs.  By key split: item = rb * nsplit + split, so
  // workgroup b (XCD b % 8) takes splits == b (mod 8).  By row block: items run row block
  // fastest within groups of 8, item = (group * nsplit + split) * 8 + rb % 8, so workgroup b
  // takes row blocks == b (mod 8).  Row blocks are padded to whole groups of 8.
  int split_i, rb;
  const bool by_row = a.by_row && (*a.by_row & 1u) != 0u;   // uniform
  if (by_row) {
    const int grp = item / (8 * a.nsplit), rem8 = item % (8 * a.nsplit);
    split_i = rem8 >> 3;
    rb = grp * 8 + (rem8 & 7);
  } else {
    split_i = item % a.nsplit;
    rb = item / a.nsplit;
  }
  if (rb * RPW >= a.nrows) return;   // padding (uniform)
  if (MODE == STORE_BLOCK && a.only_flagged && a.only_flagged[rb] == 0) return;   // uniform
  const int r_begin = a.row0 + rb * RPW;
  const int r_end = min(r_begin + RPW, a.row0 + a.nrows);

  // ---- key range of this workgroup: its split, clipped to the union of its rows' windows
  if (wave == 0) {
    int lo = INT_MAX, hi = INT_MIN, odd = 0;
    if (lane < RPW && r_begin + lane < r_end) {
      const int kst = max(a.ks[r_begin + lane], 0), ket = min(a.ke[r_begin + lane], a.L);
      if (ket > kst) { lo = kst; hi = ket; odd = kst & 7; }
    }
    for (int off = 32; off > 0; off >>= 1) {
      lo = min(lo, __shfl_xor(lo, off));
      hi = max(hi, __shfl_xor(hi, off));
      odd |= __shfl_xor(odd, off);
    }
    // any head weight of the workgroup's rows below zero (or not a number)
    int neg = 0;
    for (int i = lane; i < RPW * H; i += 64)
      if (r_begin + i / H < r_end) neg |= !(a.w[(int64_t)(r_begin + i / H) * H + i % H] >= 0.f);
    neg = __builtin_amdgcn_ballot_w64(neg != 0) != 0;
    if (lane == 0) { wg_range[0] = lo; wg_range[1] = hi; wg_range[2] = odd; wg_range[3] = neg; }
  }
  __syncthreads();
  // the launch pair splits the workgroups by their rows' head weights: the F16 form takes those
  // whose weights are all >= 0, the fp32 form the others
  if (F16 && wg_range[3] != 0) {   // uniform
    if (tid == 0) atomicMax(a.neg_seq, a.seq);
    return;
  }
  if (!F16 && wg_range[3] == 0) return;   // uniform
  int s_lo, s_hi;
  if (by_row) {
    // The row block's items share the tiles of its rows' window union evenly, in key
    // order, at least BY_ROW_MIN_TILES each: the short windows of a ragged batch then
    // spread over several workgroups instead of leaving one or two long items per block.
    const int u_lo = max(a.key_lo, wg_range[0]), u_hi = min(a.key_hi, wg_range[1]);
    const int ut0 = u_lo & ~(TK - 1);
    const int unt = u_lo < u_hi ? (u_hi - ut0 + TK - 1) / TK : 0;
    const int nact = min(a.nsplit, (unt + BY_ROW_MIN_TILES - 1) / BY_ROW_MIN_TILES);
    const int a0 = split_i < nact ? split_i * unt / nact : 0;
    const int a1 = split_i < nact ? (split_i + 1) * unt / nact : 0;
    s_lo = max(u_lo, ut0 + a0 * TK);
    s_hi = min(u_hi, ut0 + a1 * TK);
  } else {
    const int split_lo = a.key_lo + split_i * a.split;
    const int split_hi = min(split_lo + a.split, a.key_hi);
    s_lo = max(split_lo, wg_range[0]);
    s_hi = min(split_hi, wg_range[1]);
  }
  // this part's tiles of the item: [tile0, tile0 + ntiles * TK)
  const int itile0 = s_lo & ~(TK - 1);
  const int intiles = s_lo < s_hi ? (s_hi - itile0 + TK - 1) / TK : 0;
  const int pt0 = part * intiles / nparts, pt1 = (part + 1) * intiles / nparts;
  const int tile0 = itile0 + pt0 * TK;
  // Pooled blocks start at each row's ks; this part stores the blocks that start in its own
  // keys [own_lo, own_hi).  When a row's ks is not a multiple of 8, the last such block ends
  // past own_hi, so the part scores one more tile (its keys only complete that block).
  const int own_lo = max(s_lo, tile0), own_hi = min(s_hi, tile0 + (pt1 - pt0) * TK);
  const bool extend = MODE == STORE_POOL8 && wg_range[2] != 0 && pt1 > pt0 && tile0 + (pt1 - pt0) * TK < a.L;
  const int ntiles = pt1 - pt0 + (extend ? 1 : 0);
  // candidate share of this part in each of its rows' slabs
  const int share0 = part * a.caps / nparts, share = (part + 1) * a.caps / nparts - share0;
  constexpr bool cand = MODE == STORE_SLAB;
  if (cand && part == 0) {  // count words of the parts an item does not have
    for (int i = tid; i < RPW * (CAND_PARTS - nparts); i += NW * 64) {
      const int rr = r_begin + i / (CAND_PARTS - nparts);
      if (rr < r_end)
        a.ccnt[((rr - a.row0) * a.nsplit + split_i) * CAND_PARTS + nparts + i % (CAND_PARTS - nparts)] = 0;
    }
  }
  if (ntiles <= 0) {  // uniform over the workgroup: nothing to score, no candidates
    if (cand && tid < r_end - r_begin)
      a.ccnt[((r_begin - a.row0 + tid) * a.nsplit + split_i) * CAND_PARTS + part] = (uint32_t)share0 << 16;
    return;
  }

  // ---- key stages: wave w's copy `it` of a stage fills its 1 KiB block it * NW + w;
  // lane l brings 16-byte slot (it * NW + w) * 64 + l.  LDS row p of a stage holds tile
  // key 64 (p / 64) + 4 (p % 16) + (p / 16) % 4, its chunks swizzled.
  auto request = [&](int tile, int buf) {
    const int ts = tile0 + tile * TK;
#pragma unroll
    for (int it = 0; it < LPT; ++it) {
      const int slot = it * NW * 64 + tid;
      const int p = KF == 0 ? slot >> 3 : slot >> 2;
      const int chunk = KF == 0 ? (slot & 7) ^ swz8(p) : (slot & 3) ^ swz4(p);
      const int key = (p & ~63) | ((p & 15) << 2) | ((p >> 4) & 3);
      const int gk = min(ts + key, a.L - 1);
      lds_copy16(a.k + (int64_t)gk * KB + chunk * 16,
                 __builtin_amdgcn_readfirstlane(lds_addr(&kbuf[buf][(it * NW * 64 + wave * 64) * 16])));
    }
    if (wave < TK / 64)
      lds_copy4(a.k_scale + (int64_t)min(ts + tid, a.L - 1) * 4,
                __builtin_amdgcn_readfirstlane(lds_addr(&sbuf[buf][wave * 64])));
  };
  request(0, 0);
  if (ntiles > 1) request(1, 1);

  // ---- this wave's query rows: A fragments (q) and weights in registers
  const int g = lane >> 4;        // lane group: k block of A/B, row group of C
  const int n16 = lane & 15;      // A row (load) / C column (key)
  const int wr = r_begin + wave * QR;
  v8i qa[NT];
  {
    const int qi = n16 / HPT, hh = n16 % HPT;
    const int t = min(wr + qi, r_end - 1);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const uint8_t *src = a.q + ((int64_t)t * H + HPT * i + hh) * 128;
      const v4i lo = *(const v4i *)(src + 16 * g);       // k = 16 g .. 16 g + 15
      const v4i hi = *(const v4i *)(src + 64 + 16 * g);  // k = 64 + 16 g .. 64 + 16 g + 15
      qa[i] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  }
  const int qo = (4 * g) / HPT;          // query of the C rows this lane holds
  const int hbase = (4 * g) % HPT;
  const int t_out = wr + qo;
  const bool row_ok = t_out < r_end;
  int kst, ket;
  {
    const int t = min(t_out, r_end - 1);
    kst = max(a.ks[t], 0);
    ket = min(a.ke[t], a.L);
  }
  // keys this lane may store: inside its row's window and inside the workgroup range
  const int v_lo = max(kst, s_lo), v_hi = min(ket, s_hi);
  // the wave's first output row (of the launch): buffer resources cover its QR rows
  const int wrow = min(wr, a.row0 + a.nrows - 1) - a.row0;
  float thr_row = __builtin_nanf("");
  int slab = 0;  // pair offset of the lane's slab for this split, from the wave's first row's slabs
  __amdgpu_buffer_rsrc_t crsrc;
  if (cand) {
    const int rr = min(t_out, r_end - 1) - a.row0;
    thr_row = a.thr[rr];
    slab = (int)((rr - wrow) * a.cand_ld) + split_i * a.caps + share0;
    crsrc = __builtin_amdgcn_make_buffer_rsrc(a.cand + (int64_t)wrow * a.cand_ld * 2, 0, (int)(QR * a.cand_ld * 8),
                                              RSRC3);
  }
  uint32_t crow = 0;  // candidates of this lane's row so far (uniform over its 16 lanes)
  const bool writer = row_ok && (QR == 4 || (g & 1) == 0);
  const int64_t ld = a.ld;
  __amdgpu_buffer_rsrc_t orsrc =
      __builtin_amdgcn_make_buffer_rsrc(a.out + (int64_t)wrow * ld, 0, (int)(QR * ld * 4), RSRC3);
  const int obase = (t_out - a.row0 - wrow) * (int)ld;   // element offset of this lane's row

  // pooled blocks: this row's block offset inside an octet, and (lanes 14, 15) the head of the
  // block that started in the last octet of the previous batch, completed in the next one
  const int rr = kst & 7;
  float pend = -__builtin_inff();
  // 16-byte stores need a 16-byte aligned element offset
  const bool row_al = (((uintptr_t)a.out & 15) == 0) && ((ld & 3) == 0) &&
                      ((MODE == STORE_DENSE ? kst : a.key_lo) & 3) == 0;
  // exclusive key limit of this lane's stores
  const int lim = MODE == STORE_DENSE ? min(v_hi, kst + a.wcols) : v_hi;

  // The tile loop in one of two forms (template argument F16).  F16: the ReLU is the
  // clamp of a conversion to f16 and the weighted head sum runs on an f16 MFMA, two VALU
  // operations per fp8 MFMA instead of eight; the terms are rounded to f16 (relative error
  // at most 2^-11 each), so this form needs head weights >= 0, where that bounds the score's
  // relative error.  Otherwise: ReLU and head sum in fp32 on the VALU.
  {
    constexpr int SA = KF == 0 ? 25 : 19;   // |<q8, k8>| <= 128 * 448^2 < 2^25; fp8 x e2m1 < 2^19
    float wv[F16 ? 1 : NT][4];
    v8h wa[F16 ? NT / 2 : 1];
    float fback = 1.f;
    int eback = 0;
    (void)fback;
    (void)eback;
    if constexpr (F16) {
      // row weight exponents: w'' = w' 2^mrow keeps each row's largest weight in [2^13, 2^14);
      // lanes [t LPR, (t + 1) LPR) take row t's maximum over its H heads, two heads each
      constexpr int LPR = 64 / QR;
      int mexp;
      {
        const int tr = min(wr + lane / LPR, r_end - 1), h0 = (lane % LPR) * 2;
        const float w0 = a.w[(int64_t)tr * H + h0] * a.q_scale[(int64_t)tr * H + h0] * a.scale;
        const float w1 = a.w[(int64_t)tr * H + h0 + 1] * a.q_scale[(int64_t)tr * H + h0 + 1] * a.scale;
        float mx = __builtin_fmaxf(__builtin_fabsf(w0), __builtin_fabsf(w1));
        for (int off = LPR / 2; off > 0; off >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, off));
        int e = 0;
        (void)__builtin_frexpf(mx, &e);
        mexp = mx > 0.f ? 14 - e : 0;
      }
      // A of the head-sum MFMAs: row R = HPT tq + part holds query tq's weights (part 0: hi,
      // part 1: lo f16 parts of w''; other rows zero); element (g, e) of tile pair m pairs
      // with fp8 tile 2 m + e / 4, C row 4 g + e % 4, i.e. query (4 g + e % 4) / HPT and
      // head HPT (2 m + e / 4) + (4 g + e % 4) % HPT
      const int tq = n16 / HPT, part = n16 % HPT;
      const int mq = __shfl(mexp, tq * LPR);
      const int tA = min(wr + tq, r_end - 1);
#pragma unroll
      for (int m = 0; m < NT / 2; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 4 * g + e % 4, h = HPT * (2 * m + e / 4) + r % HPT;
          float v = 0.f;
          if (part < 2 && r / HPT == tq) {
            const float ww = __builtin_ldexpf(a.w[(int64_t)tA * H + h] * a.q_scale[(int64_t)tA * H + h] * a.scale, mq);
            const _Float16 whi = (_Float16)ww;
            v = part == 0 ? (float)whi : ww - (float)whi;
          }
          wa[m][e] = (_Float16)v;
        }
      // output rows: this lane's query qo, exponent 2^(SA - mrow)
      const int mo = __shfl(mexp, qo * LPR);
      eback = SA - mo;
      fback = __builtin_ldexpf(1.f, eback);
    } else {
      const int t = min(t_out, r_end - 1);
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int h = HPT * i + hbase + j;
          wv[i][j] = a.w[(int64_t)t * H + h] * a.q_scale[(int64_t)t * H + h] * a.scale;
        }
    }
    // Every value the prologue loads is in registers before the loop, so that no wait
    // for those loads is placed inside it; then stage 0 is complete.
#pragma unroll
    for (int i = 0; i < NT; ++i) in_regs(qa[i]);
    if constexpr (F16) {
#pragma unroll
      for (int m = 0; m < NT / 2; ++m) in_regs(__builtin_bit_cast(v4i, wa[m]));
      in_regs(fback);
      in_regs(eback);
    } else {
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) in_regs(wv[i][j]);
    }
    in_regs(kst);
    in_regs(ket);
    if (ntiles > 1) vm_wait_barrier<LPT>();
    else vm_wait_barrier<0>();

    // B operand of key group q = 4 b + j of a stage: LDS row p = 16 q + n16 holds key 64 b + 4 n16 + j
    auto load_bk = [&](int buf, int q) __attribute__((always_inline)) -> v8i {
      const int p = q * 16 + n16;
      if (KF == 0) {
        const int sw = swz8(p);
        const v4i lo = *(const v4i *)&kbuf[buf][p * 128 + ((g ^ sw) << 4)];
        const v4i hi = *(const v4i *)&kbuf[buf][p * 128 + (((4 + g) ^ sw) << 4)];
        return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      } else {
        const v4i v = *(const v4i *)&kbuf[buf][p * 64 + ((g ^ swz4(p)) << 4)];
        return (v8i){v.x, v.y, v.z, v.w, 0, 0, 0, 0};
      }
    };
    // f16 form: each key group's B operand is read from LDS while the group before it is
    // multiplied (the fp32 form, short of registers, reads it just before use)
    for (int it = 0; it < ntiles; ++it) {
      const int buf = it % 3;
      if (it + 2 < ntiles) request(it + 2, (it + 2) % 3);  // its buffer was last read in iteration it - 1
      const int ts = tile0 + it * TK;
      v8i bk_next = {};
      if constexpr (F16) bk_next = load_bk(buf, 0);
  #pragma unroll
      for (int b = 0; b < TK / 64; ++b) {
        const int s0 = ts + 64 * b + 4 * n16;                       // this lane's first key
        const v4i sc = *(const v4i *)&sbuf[buf][64 * b + 4 * n16];  // its 4 keys' scale words
        float val[4];
        int ebk[4] = {0, 0, 0, 0};   // MXFP4, f16 path: each key's largest block-scale code
        (void)ebk;
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          v8i bk;
          if constexpr (F16) {
            bk = bk_next;
            if (4 * b + j + 1 < TK / 16) bk_next = load_bk(buf, 4 * b + j + 1);
          } else {
            bk = load_bk(buf, 4 * b + j);
          }
          int bscale = KF == 0 ? 0 : (sc[j] >> (8 * g)) & 0xFF;
          v4f c[NT];
          if constexpr (F16) {
            // every term scaled by 2^-SA into [-1, 1]; an MXFP4 key's block scales relative to its
            // largest (the factor comes back after the head sum)
            int emax = 0;
            if (KF != 0) {
              const uint32_t w4 = (uint32_t)sc[j];
              emax = (int)max(max(w4 & 0xFFu, (w4 >> 8) & 0xFFu), max((w4 >> 16) & 0xFFu, w4 >> 24));
              bscale = max(bscale - emax + 127, 0);
              ebk[j] = emax;
            }
  #pragma unroll
            for (int i = 0; i < NT; ++i)
              c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[i], bk, (v4f){0, 0, 0, 0}, 0, KF == 0 ? 0 : 4, 0,
                                                                      127 - SA, 0, KF == 0 ? 127 : bscale);
            // ReLU and f16 rounding in one conversion, then the weighted head sum on the f16 MFMA:
            // B element (g, e) of tile pair m is C row 4 g + e % 4 of fp8 tile 2 m + e / 4 (wa
            // uses the same pairing), and C rows 4 g, 4 g + 1 collect the hi and lo weights' sums
            v4f hsum = {0, 0, 0, 0};
  #pragma unroll
            for (int m = 0; m < NT / 2; ++m) {
              const v4u bu = {cvt_relu_f16x2(c[2 * m][0], c[2 * m][1]), cvt_relu_f16x2(c[2 * m][2], c[2 * m][3]),
                              cvt_relu_f16x2(c[2 * m + 1][0], c[2 * m + 1][1]),
                              cvt_relu_f16x2(c[2 * m + 1][2], c[2 * m + 1][3])};
              hsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[m], __builtin_bit_cast(v8h, bu), hsum, 0, 0, 0);
            }
            val[j] = hsum[0] + hsum[1];
          } else {
  #pragma unroll
            for (int i = 0; i < NT; ++i) {
              if (KF == 0)
                c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[i], bk, (v4f){0, 0, 0, 0}, 0, 0, 0, 0, 0, 0);
              else
                c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[i], bk, (v4f){0, 0, 0, 0}, 0, 4, 0, 127, 0,
                                                                        bscale);
            }
            float acc = 0.f;
  #pragma unroll
            for (int i = 0; i < NT; ++i)
  #pragma unroll
              for (int jj = 0; jj < 4; ++jj) acc = __builtin_fmaf(relu(c[i][jj]), wv[i][jj], acc);
            if (QR == 2) {
              const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
              acc = __uint_as_float(r[0]) + __uint_as_float(r[1]);
            }
            val[j] = acc;
          }
        }
        if constexpr (F16) {
          // undo the scalings: 2^(SA - mrow) for the terms and weights, then the key's own scale
  #pragma unroll
          for (int j = 0; j < 4; ++j)
            val[j] = KF == 0 ? val[j] * fback * __int_as_float(sc[j]) : __builtin_ldexpf(val[j], eback + ebk[j] - 127);
        } else if (KF == 0) {
  #pragma unroll
          for (int j = 0; j < 4; ++j) val[j] *= __int_as_float(sc[j]);
        }
        if (cand) {
          // values above the row's running threshold go to its slab, in key order
          uint32_t pm = 0;
          if constexpr (KF == 0) {
            // the lane's keys s0 .. s0 + 3 inside its row's window and range as one mask per batch
            // (with fp8 keys 0.7% faster on long_ctx than testing each key; with MXFP4 keys 2% slower)
            const int wlo = min(max(v_lo - s0, 0), 4), whi = min(max(v_hi - s0, 0), 4);
            const uint32_t wm = writer && whi > wlo ? (0xFu >> (4 - whi)) & (0xFu << wlo) : 0u;
  #pragma unroll
            for (int j = 0; j < 4; ++j) pm |= (uint32_t)(val[j] > thr_row) << j;
            pm &= wm;
          } else {
  #pragma unroll
            for (int j = 0; j < 4; ++j)
              pm |= (uint32_t)(writer && s0 + j >= v_lo && s0 + j < v_hi && val[j] > thr_row) << j;
          }
          // wave-uniform tests: at high thresholds most batches have no candidate at all, and
          // a store is issued only for a j that some lane of the wave needs (lanes without a
          // candidate there, or past the slab, are dropped)
          if (__builtin_amdgcn_ballot_w64(pm != 0u)) {
            const uint32_t c = __builtin_popcount(pm);
            uint32_t tot;
            const uint32_t incl = row16_scan(c, tot);
            uint32_t pos = crow + incl - c;
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bool bit = (pm >> j) & 1u;
              if (__builtin_amdgcn_ballot_w64(bit)) {
                const v2u e = {__float_as_uint(val[j]), (uint32_t)(s0 + j)};
                __builtin_amdgcn_raw_buffer_store_b64(e, crsrc,
                                                      bit && pos < (uint32_t)share ? (slab + (int)pos) * 8 : OOB, 0, 0);
              }
              pos += bit;
            }
            crow += tot;
          }
        }
        if constexpr (MODE == STORE_DENSE || MODE == STORE_BLOCK) {
          const int col = MODE == STORE_DENSE ? s0 - kst : s0 - a.key_lo;   // column of key s0
          if (writer && row_al && s0 >= v_lo && s0 + 4 <= lim) {
            const v4u d = {__float_as_uint(val[0]), __float_as_uint(val[1]), __float_as_uint(val[2]),
                           __float_as_uint(val[3])};
            __builtin_amdgcn_raw_buffer_store_b128(d, orsrc, (obase + col) * 4, 0, 0);
          } else {
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bool ok = writer && s0 + j >= v_lo && s0 + j < lim;
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val[j]), orsrc, ok ? (obase + col + j) * 4 : OOB,
                                                    0, 0);
            }
          }
        } else if constexpr (MODE == STORE_POOL8) {
          // 8-key blocks of the row start at ks: the block starting in octet o (keys 8 o .. 8 o + 7,
          // held by lanes 2 m, 2 m + 1) is keys 8 o + r .. 8 o + r + 7, r = ks & 7.  hi: the octet's
          // in-window keys at positions >= r (the head of its block); lo: those at positions < r
          // (the tail of the block that started one octet before).
          float hi = -__builtin_inff(), lo = -__builtin_inff();
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int s = s0 + j;
            const bool in = s >= kst && s < ket;
            if (in && (s & 7) >= rr) hi = __builtin_fmaxf(hi, val[j]);
            if (in && (s & 7) < rr) lo = __builtin_fmaxf(lo, val[j]);
          }
          hi = __builtin_fmaxf(hi, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(hi), 0xB1, 0xF, 0xF, false)));
          lo = __builtin_fmaxf(lo, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(lo), 0xB1, 0xF, 0xF, false)));
          // the next octet's tail: two lanes up (row rotate right by 14); lanes 14, 15 receive the
          // tail of this batch's first octet, which completes the block they held back last batch
          const float nlo = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(lo), 0x12E, 0xF, 0xF, false));
          int bo = s0 >> 3;   // octet of the block start stored now
          float m = rr ? __builtin_fmaxf(hi, nlo) : hi;
          if (rr && n16 >= 14) {
            m = __builtin_fmaxf(pend, nlo);
            bo -= 8;
            pend = hi;
          }
          const int bs = 8 * bo + rr;                  // the block's first key
          const int col = bo - (a.key_lo >> 3);
          const bool st = writer && (n16 & 1) == 0 && bs >= kst && bs < ket && bs >= own_lo && bs < own_hi &&
                          col < a.wcols;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), orsrc, st ? (obase + col) * 4 : OOB, 0, 0);
        }
      }
      // stage it + 1 is complete once no more than the memory operations issued after its
      // request are outstanding: >= ST stores of iteration it - 1, stage it + 2's request
      // (>= LPT copies), >= ST stores of this iteration
      if (it + 1 < ntiles) {
        if (it + 2 < ntiles) {
          if (it > 0) vm_wait_barrier<2 * ST + LPT>();
          else vm_wait_barrier<ST + LPT>();
        } else {
          if (it > 0) vm_wait_barrier<2 * ST>();
          else vm_wait_barrier<ST>();
        }
      }
    }
  }
  if (cand && writer && n16 == 0)
    a.ccnt[((int64_t)(t_out - a.row0) * a.nsplit + split_i) * CAND_PARTS + part] =
        ((uint32_t)share0 << 16) | (crow > (uint32_t)share ? CAND_OVER : crow);
}

// Workgroups of one kernel the current device runs at once (CUs x workgroups per CU),
// queried once per device and kernel.
// Host threads may call concurrently: entries are atomics, and a race only repeats the query.
template <class Kern>
int resident_workgroups(Kern kern, int threads) {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) != hipSuccess)
      return 0;
    n = cus * per_cu;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

constexpr int NW_LAUNCH = 4;   // 4 waves: up to 3 workgroups per CU, so a stage barrier never idles the CU

template <int KF, int H, int MODE, bool F16>
hipError_t launch4(const LogitsArgs &a0, hipStream_t s) {
  constexpr int NW = NW_LAUNCH;
  constexpr int RPW = NW * (128 / H);
  auto kern = logits_kernel<KF, H, MODE, NW, F16>;
  const int nrb = (a0.nrows + RPW - 1) / RPW;
  const int64_t items = (int64_t)((nrb + 7) / 8) * 8 * a0.nsplit;   // row blocks padded to whole groups of 8
  if (items <= 0) return hipSuccess;
  // Whole items fill as many complete waves of resident workgroups as they can; the
  // remainder is cut into parts so that the last waves span the machine as well: into the
  // part count p <= CAND_PARTS whose ceil(rem p / slots) / p item-lengths of tail is
  // shortest (rem = 512 on 768 slots: 3 parts, 2/3 of an item instead of a whole one).
  LogitsArgs a = a0;
  const int64_t slots = resident_workgroups(kern, NW * 64);
  const int64_t full_waves = slots > 0 ? items / slots : items;
  const int64_t rem = items - full_waves * slots;
  a.parts = 1;
  if (rem > 0 && slots > 0) {
    int64_t bw = (rem + slots - 1) / slots, bp = 1;   // tail = bw / bp item-lengths
    for (int64_t p = 2; p <= CAND_PARTS; ++p) {
      const int64_t w = (rem * p + slots - 1) / slots;
      if (w * bp < bw * p) { bw = w; bp = p; }
    }
    a.parts = (int)bp;
  }
  a.nfull = (int)(items - rem);
  const int64_t grid = a.nfull + rem * a.parts;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

// The launch pair marker word, one per device (its address looked up once per device).
static __device__ unsigned long long neg_seq_word;
std::atomic<unsigned long long *> neg_seq_on_device[64];
std::atomic<unsigned long long> neg_seq_next{0};

hipError_t neg_seq_address(unsigned long long **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  unsigned long long *p = neg_seq_on_device[dev].load(std::memory_order_acquire);
  if (!p) {
    void *v = nullptr;
    e = hipGetSymbolAddress(&v, HIP_SYMBOL(neg_seq_word));
    if (e != hipSuccess) return e;
    if (!v) return hipErrorInvalidSymbol;
    p = (unsigned long long *)v;
    neg_seq_on_device[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

// Both forms over the same grid: each workgroup works in exactly one of them.  The fp32 form
// leaves at once unless the f16 form marked the pair.  Concurrent launch pairs on one device
// (other streams) can only make an fp32 form look at its rows' weights needlessly: the word
// only grows, and a pair's own mark is in place before its fp32 form starts.
template <int KF, int H, int MODE>
hipError_t launch3(const LogitsArgs &a0, hipStream_t s) {
  LogitsArgs a = a0;
  hipError_t e = neg_seq_address(&a.neg_seq);
  if (e != hipSuccess) return e;
  a.seq = neg_seq_next.fetch_add(1, std::memory_order_relaxed) + 1;
  e = launch4<KF, H, MODE, true>(a, s);
  if (e != hipSuccess) return e;
  return launch4<KF, H, MODE, false>(a, s);
}

template <int KF, int H>
hipError_t launch2(const LogitsArgs &a, int mode, hipStream_t s) {
  switch (mode) {
    case STORE_DENSE: return launch3<KF, H, STORE_DENSE>(a, s);
    case STORE_BLOCK: return launch3<KF, H, STORE_BLOCK>(a, s);
    case STORE_SLAB: return launch3<KF, H, STORE_SLAB>(a, s);
    default: return launch3<KF, H, STORE_POOL8>(a, s);
  }
}

}  // namespace

int logits_rows_per_workgroup(int H) { return NW_LAUNCH * (128 / H); }

hipError_t launch_logits(const LogitsArgs &a, int k_fmt, int H, int mode, hipStream_t s) {
  if (k_fmt == 0) return H == 32 ? launch2<0, 32>(a, mode, s) : launch2<0, 64>(a, mode, s);
  return H == 32 ? launch2<1, 32>(a, mode, s) : launch2<1, 64>(a, mode, s);
}

}  // namespace idx
