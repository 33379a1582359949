// Tiled block-sparse prefill attention for gfx950 (MiniCPM4 paper summary, section 2.1.3:
// each token attends only to its most relevant KV blocks; FlashAttention-style online
// softmax).
//
// Design (one workgroup = 8 waves = one tile of T consecutive query tokens of one sequence and
// one KV head: T = 24 in the sparse forward at groups of 16 heads and in the window form, 32 in
// the sparse forward at groups of 8 (64 at head_dim 64), 16 in the gradient form):
//   * Union: the tile's T selected-block lists are OR-ed into a per-block T-bit token mask in
//     LDS and compacted into a list of (block, mask).  Each union block's K and V (64 keys x d,
//     bf16) are staged into LDS once for all tokens that chose it.  The forward and gradient
//     forms stream the list in the order of the waves' progress (each wave's needed blocks,
//     ranked r = 0 .. n_w - 1, get the key (r + 1/2) / n_w; an entry takes its waves' largest
//     key), so that any stretch of the stream holds about equal work for every wave and fewer
//     waves idle at the head of the ring; the order stays close to ascending block order.
//   * Staging: global_load_lds (16 B per lane, straight to LDS, no registers) into a ring of
//     NS slots, block u in slot u % NS.  K is stored row-major with the 16-byte chunks of row r
//     XOR-swizzled by kswz(r), so that an A-operand read spans all banks; V in the unit order
//     its transposing reads want.  The last wave to finish with a slot (an LDS counter against
//     the number of waves whose tokens chose the block) refills it with block u + NS and
//     raises the slot's ready word once the loads have landed (at raised wave priority until
//     then); waits poll that word, bounded.
//   * Compute: wave w owns tokens TPW*w .. TPW*w + TPW - 1 (T / 8 of them; registers: Q operand,
//     O accumulator, running max and sum per 16-column group, a group holding one token's 16
//     heads or two tokens' 8).  For every union block it processes only its groups with a
//     token whose mask bit is set:
//       S^T = K Q^T   16 keys x 16 columns per v_mfma_f32_16x16x32_bf16 (A = K from LDS)
//       online softmax over the 64 keys (exp2; the running max moves only when a block's max
//                     exceeds it by more than kLazy, decided for the whole wave)
//       O  += P V     16 heads x 16 dims per MFMA; B = V read with ds_read_b64_tr_b16, which
//                     transposes 4x16 bf16 tiles across each 16-lane group, so V needs no
//                     transposed copy.  The key order inside each 32-key step makes the
//                     S^T fragment a lane holds exactly its P operand.
//   * Scheduling: launches go in rounds of one workgroup per compute unit; in a round each XCD
//     (blockIdx % 8) runs a group of consecutive tiles of one (sequence, KV head), which select
//     from the same blocks and share that XCD's L2.  Groups are taken by their position in the
//     sequence, highest first, so that the eight groups of a round take about as long.
#include <algorithm>
#include <atomic>

#include "dpp.h"
#include "internal.h"

namespace infllm2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kT = 16;            // query tokens per workgroup of the gradient form
constexpr int kTW = 24;           // ... of the window form (3 tokens per wave: 13.2 ms at 128K
                                  // and window 6144, against 13.8 with 16)
constexpr int kWaves = 8;         // their waves per workgroup (tokens per wave = kT / kWaves)
constexpr int kTF = 24;           // query tokens per workgroup of the sparse forward (G = 16)
constexpr int kTF8 = 32;          // ... at G = 8 (two tokens' heads stacked per MFMA group)
constexpr int kTF8S = 64;         // ... at G = 8 and head_dim 64 (the smaller accumulators fit)
constexpr int kWavesF = 8;        // its waves (two per SIMD, TF / 8 tokens each)
constexpr int kMaxUnion = 2048;   // reachable blocks per tile handled by this kernel
constexpr int kRoundsPerLaunch = 3;  // rounds of the tile schedule per kernel launch
constexpr float kLazy = 8.f;      // log2 headroom before the running max is moved
constexpr int kSpinLimit = 1 << 20;  // bounded waits (about 30 ms): a protocol error never hangs
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3 for gfx9-family raw buffers

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most `later` blocks of PER loads each are still in flight (later clamped to
// MAXL): the oldest block has landed in LDS.
template <int PER, int MAXL>
__device__ __forceinline__ void wait_blocks(int later) {
  if constexpr (MAXL > 0) {
    if (later >= MAXL) {
      wait_vmcnt<MAXL * PER>();
      return;
    }
    wait_blocks<PER, MAXL - 1>(later);
  } else {
    wait_vmcnt<0>();
  }
}

__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// XOR swizzle of the 16-byte chunk index within a row (bijective per row).
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  return ((r & 3) | ((r >> 1) & 12)) & (CPR - 1);
}

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// Transposing reads of V for 2*NH MFMA B-operands (tiles n = 0..NH-1, h = 0..1) at immediate
// offsets 512*(2n + h) from `addr`, waited for inside the same asm statement (the compiler does
// not track loads it cannot see).  vt[n][h] = 4 bf16: V[32s + 8*q4 + 4h + 0..3][16n' + c16].
template <int NH>
__device__ __forceinline__ void read_v_half(uint32_t addr, uint64_t (&vt)[NH][2]);

template <>
__device__ __forceinline__ void read_v_half<4>(uint32_t addr, uint64_t (&vt)[4][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %8 offset:512\n"
      "ds_read_b64_tr_b16 %2, %8 offset:1024\n"
      "ds_read_b64_tr_b16 %3, %8 offset:1536\n"
      "ds_read_b64_tr_b16 %4, %8 offset:2048\n"
      "ds_read_b64_tr_b16 %5, %8 offset:2560\n"
      "ds_read_b64_tr_b16 %6, %8 offset:3072\n"
      "ds_read_b64_tr_b16 %7, %8 offset:3584\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(vt[0][0]), "=&v"(vt[0][1]), "=&v"(vt[1][0]), "=&v"(vt[1][1]),
        "=&v"(vt[2][0]), "=&v"(vt[2][1]), "=&v"(vt[3][0]), "=&v"(vt[3][1])
      : "v"(addr)
      : "memory");
}

template <>
__device__ __forceinline__ void read_v_half<8>(uint32_t addr, uint64_t (&vt)[8][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n"
      "ds_read_b64_tr_b16 %1, %16 offset:512\n"
      "ds_read_b64_tr_b16 %2, %16 offset:1024\n"
      "ds_read_b64_tr_b16 %3, %16 offset:1536\n"
      "ds_read_b64_tr_b16 %4, %16 offset:2048\n"
      "ds_read_b64_tr_b16 %5, %16 offset:2560\n"
      "ds_read_b64_tr_b16 %6, %16 offset:3072\n"
      "ds_read_b64_tr_b16 %7, %16 offset:3584\n"
      "ds_read_b64_tr_b16 %8, %16 offset:4096\n"
      "ds_read_b64_tr_b16 %9, %16 offset:4608\n"
      "ds_read_b64_tr_b16 %10, %16 offset:5120\n"
      "ds_read_b64_tr_b16 %11, %16 offset:5632\n"
      "ds_read_b64_tr_b16 %12, %16 offset:6144\n"
      "ds_read_b64_tr_b16 %13, %16 offset:6656\n"
      "ds_read_b64_tr_b16 %14, %16 offset:7168\n"
      "ds_read_b64_tr_b16 %15, %16 offset:7680\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(vt[0][0]), "=&v"(vt[0][1]), "=&v"(vt[1][0]), "=&v"(vt[1][1]),
        "=&v"(vt[2][0]), "=&v"(vt[2][1]), "=&v"(vt[3][0]), "=&v"(vt[3][1]),
        "=&v"(vt[4][0]), "=&v"(vt[4][1]), "=&v"(vt[5][0]), "=&v"(vt[5][1]),
        "=&v"(vt[6][0]), "=&v"(vt[6][1]), "=&v"(vt[7][0]), "=&v"(vt[7][1])
      : "v"(addr)
      : "memory");
}

template <>
__device__ __forceinline__ void read_v_half<2>(uint32_t addr, uint64_t (&vt)[2][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n"
      "ds_read_b64_tr_b16 %1, %4 offset:512\n"
      "ds_read_b64_tr_b16 %2, %4 offset:1024\n"
      "ds_read_b64_tr_b16 %3, %4 offset:1536\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(vt[0][0]), "=&v"(vt[0][1]), "=&v"(vt[1][0]), "=&v"(vt[1][1])
      : "v"(addr)
      : "memory");
}

// LDS read for polling flags written by other waves.  Written as one asm statement that waits
// for its own result: an atomic load would make the compiler first wait for every LDS-DMA load
// this wave has in flight.
__device__ __forceinline__ int lds_peek(const int* p) {
  int v;
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)p));
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}

__device__ __forceinline__ int lds_load(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(int* p, int x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Chunk swizzle of row-major K rows: for the 16 rows of one A-operand read (8(c16/4) + c16%4
// plus a multiple of 4) it is distinct per row parity class, so the 16 lanes of a read hit
// distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (D == 128) return ((row >> 1) & 12) | (row & 3);
  else return ((row >> 2) & 6) | ((row >> 1) & 1);
}

// Scheduling groups for NK k-steps of PER LDS reads feeding PER MFMAs each: the reads of the
// first AHEAD k-steps, then per k-step its MFMAs, each followed by one read AHEAD k-steps on.
template <int NK, int PER, int AHEAD>
__device__ __forceinline__ void sched_reads_ahead() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  __builtin_amdgcn_sched_group_barrier(kDsRead, AHEAD * PER, 0);
#pragma unroll
  for (int ks = 0; ks < NK; ++ks)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      if (ks + AHEAD < NK) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
    }
}

// Work items of the tile launches are groups of gs consecutive tiles of one (sequence, KV head),
// the tiles one XCD runs in one round.  Group j of a sequence (tiles gs*j .. gs*j + gs - 1) is at
// level j; groups are numbered from the highest level down, then by sequence, then by KV head,
// so that the eight groups of a round lie at about the same position in their sequences and take
// about as long (a tile's work grows with its position: more reachable blocks).  Finds the
// sequence, KV head and level of group gi; false past the last group.  groups(s) is the number
// of groups of sequence s.  Every lane of a full wave calls it with the same gi; the results are
// wave-uniform.  One pass over the sequences per distinct group count.
template <typename F>
__device__ __forceinline__ bool locate_group(const SeqTable& t, int gi, int hkv, F groups, int& b,
                                             int& kvh, int& level) {
  const int lane = threadIdx.x & 63;
  int lev = -1;                                   // the highest level
  for (int base = 0; base < t.n; base += 64) {
    const int gl = base + lane < t.n ? groups(base + lane) : 0;
    lev = max(lev, static_cast<int>(wave_max_u32(static_cast<uint32_t>(gl))) - 1);
  }
  long long acc = 0;                              // groups above level lev
  while (lev >= 0) {
    // c groups at each of the levels nxt + 1 .. lev (the same sequences have a group there)
    int c = 0, nxt = -1;
    for (int base = 0; base < t.n; base += 64) {
      const int gl = base + lane < t.n ? groups(base + lane) : 0;
      c += __popcll(__ballot(gl > lev));
      nxt = max(nxt, static_cast<int>(wave_max_u32(static_cast<uint32_t>(gl <= lev ? gl : 0))) - 1);
    }
    c *= hkv;
    const long long span = static_cast<long long>(lev - nxt) * c;
    if (gi - acc < span) {
      const int off = static_cast<int>(gi - acc);
      level = uniform(lev - off / c);
      const int r = off % c;
      kvh = uniform(r % hkv);
      int rs = r / hkv;                           // the rs-th sequence having a group at lev
      for (int base = 0; base < t.n; base += 64) {
        const int gl = base + lane < t.n ? groups(base + lane) : 0;
        const unsigned long long m = __ballot(gl > lev);
        const int pc = __popcll(m);
        if (rs < pc) {
          const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
          b = uniform(base + __ffsll(static_cast<unsigned long long>(__ballot(gl > lev && below == rs))) - 1);
          return true;
        }
        rs -= pc;
      }
      return false;
    }
    acc += span;
    lev = nxt;
  }
  return false;
}

// Number of waves (groups of TPW consecutive token bits) with any bit set in a token mask.
template <int TPW, int NW, typename M>
__device__ __forceinline__ int count_wave_groups(M m) {
  int n = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) n += ((m >> (TPW * w)) & ((M{1} << TPW) - 1u)) != 0u;
  return n;
}

// BWD = false: the attention itself (writes out, lse).  BWD = true: dQ for upstream gradient
// dout, given the forward's lse (natural log) and delta[row, head] = dout . out; the slot then
// holds V in the same A-operand order as K, and K's transposing reads come from K's own copy.
// WIN = true (forward only): sliding-window attention over keys pos - g.window < j <= pos; the
// blocks come from the positions instead of idx.
// ORD: stream the union in the order of the waves' normalised progress instead of ascending
// block order.
template <int D, int G, int NS, int NW, int TPW, bool BWD, bool WIN = false, bool ORD = false>
__global__ void __launch_bounds__(64 * NW, 1)
attn_tile(Geom g, SeqTable t, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
          const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
          uint16_t* __restrict__ out, float* __restrict__ lse, int group_base,
          const uint16_t* __restrict__ dout, const float* __restrict__ lse_in,
          const float* __restrict__ delta, float* __restrict__ dq) {
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int MAT = 64 * D * 2;            // bytes of one 64-key matrix
  constexpr int NTHR = 64 * NW;
  constexpr int T = NW * TPW;                // query tokens of the tile
  // tokens per 16-column MFMA group: two tokens' 8 heads share the columns in the forward form
  constexpr int TPC = (!BWD && !WIN && G < 16) ? 16 / G : 1;
  constexpr int CG = TPW / TPC;              // column groups per wave
  static_assert(TPC * G == 16 || TPC == 1, "a column group is one token or fills 16 columns");
  static_assert(TPW % TPC == 0, "whole column groups per wave");
  // token masks: 32 bits, or 64 for tiles of more than 32 tokens
  using MaskT = typename std::conditional<(T > 32), unsigned long long, uint32_t>::type;
  constexpr int MB = 8 * static_cast<int>(sizeof(MaskT));
  static_assert(T <= MB && MB % T != 1, "tile of at most 64 tokens");
  constexpr int MPW = (T & (T - 1)) == 0 ? MB / T : 1;  // token masks per bitmap word
  constexpr MaskT TMASK = T == MB ? ~MaskT{0} : (MaskT{1} << (T % MB)) - 1u;
  __shared__ __attribute__((aligned(16))) unsigned char ring[NS][2][MAT];
  // the bitmap of the union build lives at the end of the ring, which is free until staging
  // (the stream-order sort uses its start)
  constexpr int BITMAP_BYTES = kMaxUnion / MPW * static_cast<int>(sizeof(MaskT));
  static_assert(BITMAP_BYTES + 4 * kMaxUnion <= NS * 2 * MAT, "bitmap and sort keys fit the ring");
  MaskT* const bitmap = reinterpret_cast<MaskT*>(&ring[0][0][0] + NS * 2 * MAT - BITMAP_BYTES);
  __shared__ MaskT umask[kMaxUnion];         // union list: token mask of entry u
  __shared__ uint16_t ublk[kMaxUnion];       //             its block index
  __shared__ int wave_tot[NW];
  __shared__ int ready[NS];
  __shared__ int done[NS];

  // XCD-aware: workgroup b runs on XCD b % 8; the launch holds kRoundsPerLaunch rounds of 8
  // groups of gs tiles, round r of it (b / 8gs) giving group group_base + 8r + b % 8 to that XCD,
  // whose workgroups take the group's consecutive tiles
  const int gs = static_cast<int>(gridDim.x) / (8 * kRoundsPerLaunch);
  auto groups_of = [&](int s) { return ((t.q_len[s] + T - 1) / T + gs - 1) / gs; };
  int b, kvh, level;
  const int bx = static_cast<int>(blockIdx.x);
  if (!locate_group(t, group_base + 8 * (bx / (8 * gs)) + bx % 8, g.Hkv, groups_of, b, kvh, level))
    return;
  const int lt = level * gs + (bx / 8) % gs;
  const Seq sq = load_seq(t, b);
  if (lt * T >= sq.q_len) return;
  const int r0 = lt * T;
  const int nq = min(T, sq.q_len - r0);
  const int row0 = sq.q_start + r0;
  const int pos0 = sq.q_pos0 + r0;
  const int kv0 = sq.kv_start;
  const int kv_len = sq.kv_len;
  const int nbt = (pos0 + nq - 1) / 64 + 1;  // reachable blocks of the tile (<= kMaxUnion)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int Hq = g.Hq, Hkv = g.Hkv;

  // ---- union of the tile's selected blocks
  for (int e = tid; e < (nbt + MPW - 1) / MPW; e += NTHR) bitmap[e] = MaskT{0};
  __syncthreads();
  if constexpr (WIN) {
    // token tok needs the blocks meeting [pos - window + 1, pos]
    const int blo = max(0, pos0 - g.window + 1) / 64;
    for (int blk = blo + tid; blk < nbt; blk += NTHR) {
      MaskT m = 0u;
      for (int tok = 0; tok < nq; ++tok) {
        const int pos = pos0 + tok;
        if (64 * blk <= pos && 64 * blk + 63 > pos - g.window) m |= MaskT{1} << tok;
      }
      if (m != 0u) atomicOr(&bitmap[blk / MPW], m << (T * (blk % MPW)));
    }
  } else {
    for (int e = tid; e < nq * g.topk; e += NTHR) {
      const int tok = e / g.topk;
      const int blk = idx[(static_cast<size_t>(row0 + tok) * Hkv + kvh) * g.topk + (e - tok * g.topk)];
      if (blk >= 0) atomicOr(&bitmap[blk / MPW], (MaskT{1} << tok) << (T * (blk % MPW)));
    }
  }
  __syncthreads();
  {
    // each thread compacts KPT consecutive blocks; block-wide exclusive scan of the counts
    constexpr int KPT = kMaxUnion / NTHR;
    const int b0 = tid * KPT;
    MaskT m8[KPT];
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int blk = b0 + e;
      m8[e] = blk < nbt ? (bitmap[blk / MPW] >> (T * (blk % MPW))) & TMASK : 0u;
      cnt += m8[e] != 0u;
    }
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wave_tot[w] = incl;
    __syncthreads();
    int base = incl - cnt;
    for (int ww = 0; ww < w; ++ww) base += wave_tot[ww];
#pragma unroll
    for (int e = 0; e < KPT; ++e)
      if (m8[e] != 0u) {
        umask[base] = m8[e];
        ublk[base] = static_cast<uint16_t>(b0 + e);
        ++base;
      }
  }
  __syncthreads();
  int n_union = 0;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) n_union += wave_tot[ww];

  if constexpr (ORD) {
    // Stream order: merge the waves' lists of needed blocks by normalised progress, so that
    // every stretch of the stream holds about as much work for each wave.  Entry u needed by
    // wave w as its r-th of n_w blocks gets the key (r + 1/2) / n_w; an entry takes the largest
    // key over its waves, ties by block order.  Sorted (bitonic) in the ring's memory, which is
    // free until staging starts.
    uint32_t* skey = reinterpret_cast<uint32_t*>(&ring[0][0][0]);
    int npow2 = 1;
    while (npow2 < n_union) npow2 <<= 1;
    for (int e = tid; e < npow2; e += NTHR) skey[e] = e < n_union ? 0u : 0xFFFFFFFFu;
    __syncthreads();
    {
      const MaskT wbits = ((MaskT{1} << TPW) - 1u) << (TPW * w);
      int n_w = 0;
      for (int base = 0; base < n_union; base += 64) {
        const bool nd = base + lane < n_union && (umask[base + lane] & wbits) != 0u;
        n_w += __builtin_popcountll(__ballot(nd));
      }
      int rank = 0;
      for (int base = 0; base < n_union; base += 64) {
        const int u = base + lane;
        const bool nd = u < n_union && (umask[u] & wbits) != 0u;
        const unsigned long long bal = __ballot(nd);
        if (nd) {
          const int r = rank + __builtin_popcountll(bal & ((1ull << lane) - 1ull));
          const uint32_t key = static_cast<uint32_t>(((2u * r + 1u) << 19) / static_cast<uint32_t>(n_w));
          atomicMax(&skey[u], (key << 11) | static_cast<uint32_t>(u));
        }
        rank += __builtin_popcountll(bal);
      }
    }
    __syncthreads();
    for (int kk = 2; kk <= npow2; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < npow2; i += NTHR) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint32_t a = skey[i], c = skey[ixj];
            if ((a > c) == ((i & kk) == 0)) {
              skey[i] = c;
              skey[ixj] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    constexpr int EPT = kMaxUnion / NTHR;
    MaskT pm[EPT];
    uint16_t pb[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = tid + e * NTHR;
      if (i < n_union) {
        const int u = static_cast<int>(skey[i] & 2047u);
        pm[e] = umask[u];
        pb[e] = ublk[u];
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = tid + e * NTHR;
      if (i < n_union) {
        umask[i] = pm[e];
        ublk[i] = pb[e];
      }
    }
    __syncthreads();
  }

  // ---- staging.  global_load_lds writes lane l's 16 bytes at LDS unit base+l, and each lane
  // picks its own source, so both matrices are stored in the order their readers want:
  //   K (forward): row-major, load J covering rows RPI*J .. RPI*J + RPI-1 whole (full-row
  //      reads stream several times faster than short segments), row r's chunk c stored at
  //      position c ^ kswz(r), which spreads the 16 rows of one A-operand read over all banks;
  //   K (gradient form): unit 64*J + lane holds the A-operand chunk that lane reads for MFMA
  //      step J, i.e. J = (2s + tp)*KS + ks, row 32s + 8(c16/4) + 4tp + c16%4, chunk 4ks + q4
  //      (its transposing reads for dQ rely on this order); V then is row-major like K above;
  //   V: unit 32*((s*NT + n)*2 + h) + 8q + 2j + a1 holds row 32s + 8q + 4h + j, chunk 2n + a1,
  //      so every transposing read of (s, n, h) covers 512 contiguous bytes.
  // Both offsets split into a lane part (VGPR) and a part that depends only on the load J.
  const int rowstride = Hkv * D;                                // elements per key row
  const int k_lrow = 8 * (c16 >> 2) + (c16 & 3);
  const int v_lrow = 8 * ((lane & 31) >> 3) + 4 * (lane >> 5) + ((lane >> 1) & 3);
  const int k_lane_off = k_lrow * rowstride + 8 * q4;
  const int v_lane_off = v_lrow * rowstride + 8 * (lane & 1);
  const uint16_t* kbase = k + static_cast<size_t>(kv0) * rowstride + static_cast<size_t>(kvh) * D;
  const uint16_t* vbase = v + static_cast<size_t>(kv0) * rowstride + static_cast<size_t>(kvh) * D;
  // Loads J in [j0, CPR) step dj of union block u into ring slot `slot`.  Full blocks use buffer
  // loads: a uniform base (descriptor), the lane's fixed byte offset and a scalar offset per J,
  // so no per-load address arithmetic.  The ragged last block clamps rows per lane instead.
  const int k_lane_bytes = 2 * k_lane_off;
  const int v_lane_bytes = 2 * v_lane_off;
  constexpr bool KROW = !BWD;
  constexpr int RPI = 64 / CPR;                                 // K rows per load (row-major)
  const int kr_lane = lane / CPR;
  const int kp_lane = lane % CPR;
  auto produce = [&](int u, int slot, int j0, int dj) {
    const int key0 = __builtin_amdgcn_readfirstlane(static_cast<int>(ublk[u])) * 64;
    const bool tail = key0 + 64 > kv_len;
    const uint16_t* kb = kbase + static_cast<size_t>(key0) * rowstride;
    const uint16_t* vb = vbase + static_cast<size_t>(key0) * rowstride;
    if (!tail) {
      const int nbytes = (63 * rowstride + D) * 2;               // the block's rows of this head
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(kb), 0, nbytes, kBufferWord3);
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(vb), 0, nbytes, kBufferWord3);
      for (int J = j0; J < CPR; J += dj) {
        const int krow0 = 32 * (J / (2 * KS)) + 4 * ((J / KS) % 2);
        const int vrow0 = 32 * (J / NT);
        const int ks_off = (krow0 * rowstride + 32 * (J % KS)) * 2;
        const int vs_off = (vrow0 * rowstride + 16 * (J % NT)) * 2;
        if constexpr (KROW) {
          const int c = kp_lane ^ kswz<D>(RPI * J + kr_lane);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(&ring[slot][0][J * 1024]), 16,
                                                   (kr_lane * rowstride + 8 * c) * 2,
                                                   RPI * J * rowstride * 2, 0, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(&ring[slot][0][J * 1024]), 16,
                                                   k_lane_bytes, ks_off, 0, 0);
        }
        if constexpr (BWD) {       // V row-major like the forward's K (it is an A operand here)
          const int c = kp_lane ^ kswz<D>(RPI * J + kr_lane);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(&ring[slot][1][J * 1024]), 16,
                                                   (kr_lane * rowstride + 8 * c) * 2,
                                                   RPI * J * rowstride * 2, 0, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(&ring[slot][1][J * 1024]), 16,
                                                   v_lane_bytes, vs_off, 0, 0);
        }
      }
      return;
    }
    const int last = kv_len - 1 - key0;
    for (int J = j0; J < CPR; J += dj) {
      const int krow0 = 32 * (J / (2 * KS)) + 4 * ((J / KS) % 2);
      const int vrow0 = 32 * (J / NT);
      int ko = k_lane_off + krow0 * rowstride + 32 * (J % KS);
      int vo = v_lane_off + vrow0 * rowstride + 16 * (J % NT);
      const int kr = krow0 + k_lrow, vr = vrow0 + v_lrow;
      ko += ((kr < last ? kr : last) - kr) * rowstride;
      vo += ((vr < last ? vr : last) - vr) * rowstride;
      if constexpr (KROW) {
        const int row = RPI * J + kr_lane;
        ko = (row < last ? row : last) * rowstride + 8 * (kp_lane ^ kswz<D>(row));
      }
      __builtin_amdgcn_global_load_lds(kb + ko, (lds_void*)(&ring[slot][0][J * 1024]), 16, 0, 0);
      if constexpr (BWD) {
        const int row = RPI * J + kr_lane;
        const int vo_r = (row < last ? row : last) * rowstride + 8 * (kp_lane ^ kswz<D>(row));
        __builtin_amdgcn_global_load_lds(vb + vo_r, (lds_void*)(&ring[slot][1][J * 1024]), 16, 0, 0);
      } else {
        __builtin_amdgcn_global_load_lds(vb + vo, (lds_void*)(&ring[slot][1][J * 1024]), 16, 0, 0);
      }
    }
  };

  // ---- per-column-group state.  The 16 MFMA columns of a group hold TPC tokens' G heads
  // (TPC = 16 / G stacked tokens in the forward form at G = 8, else 1): column c16 is token
  // TPW*w + TPC*tt + c16 / G, head c16 % G.  m_run is shared by the 4 lanes of a column (log2
  // units, possibly stale by < kLazy); l_run is this lane's partial row sum.
  // Backward: dof = dout in the same B-operand order as q, lse2 = lse * log2(e) and dl = delta
  // for head c16 (+inf / 0 on unused lanes, so their probabilities are 0), o accumulates the
  // dQ^T tiles (dims x heads).
  bf16x8 qf[CG][KS];
  bf16x8 dof[CG][KS];
  f32x4 o[CG][NT];
  float m_run[CG], l_run[CG];
  float lse2[CG], dl[CG];
  const int ct = TPC == 1 ? 0 : c16 / G;     // the lane column's token within its group
  const int hd = TPC == 1 ? c16 : c16 % G;   // ... and its head
#pragma unroll
  for (int tt = 0; tt < CG; ++tt) {
    const int tw = TPW * w + TPC * tt + ct;
    m_run[tt] = -INFINITY;
    l_run[tt] = 0.f;
#pragma unroll
    for (int n = 0; n < NT; ++n) o[tt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool live = tw < nq && hd < G;
    const size_t hrow = static_cast<size_t>(row0 + tw) * Hq + kvh * G + hd;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[tt][ks] = live ? *reinterpret_cast<const bf16x8*>(q + hrow * D + 32 * ks + 8 * q4)
                        : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
      if constexpr (BWD)
        dof[tt][ks] = live ? *reinterpret_cast<const bf16x8*>(dout + hrow * D + 32 * ks + 8 * q4)
                           : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
    if constexpr (BWD) {
      lse2[tt] = live ? lse_in[hrow] * kLog2e : INFINITY;
      dl[tt] = live ? delta[hrow] : 0.f;
    }
  }
  // the first NS union blocks are loaded by all waves together
  for (int u = 0; u < NS && u < n_union; ++u) produce(u, u, w, NW);
  if (tid < NS) {
    ready[tid] = tid < n_union ? tid : -1;
    done[tid] = 0;
  }
  wait_vmcnt<0>();
  __syncthreads();

  const float qscale = g.scale * kLog2e;
  const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&ring[0][0][0]));
  const uint32_t k_lane = ring_lds + 16 * lane;                                 // + slot, + 1KB*J
  // row-major K: lane's A-operand chunk for k-step ks of row 8(c16/4) + c16%4 (+ 32s + 4tp)
  uint32_t kofs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int krl = 8 * (c16 >> 2) + (c16 & 3);
    kofs[ks] = ring_lds + static_cast<uint32_t>(krl * 2 * D + 16 * ((4 * ks + q4) ^ kswz<D>(krl)));
  }
  // Transposing reads: forward, V (matrix 1, stored for them); backward, K (matrix 0, stored in
  // A-operand order).  In K's order, keys 32s + 8q + 4h + (0..3), dims 16n + 4c .. 4c+3 sit in
  // unit 64((2s + h)KS + n/2) + 16(2(n%2) + c/2) + 4q + (0..3), half c%2, so a lane's reads of
  // (h, n) are 512 (NT h + n) bytes apart and each read covers 512 contiguous bytes.
  const uint32_t v_lane =
      BWD ? ring_lds + 256 * ((c16 & 3) >> 1) + 64 * q4 + 16 * (c16 >> 2) + 8 * (c16 & 1)
          : ring_lds + MAT + 16 * (8 * q4 + 2 * (c16 >> 2) + ((c16 & 3) >> 1)) + 8 * (c16 & 1);

  // ---- main loop.  Each wave walks the union list in stream order and works only on blocks
  // its tokens chose.  Slot u % NS holds stream entry u once ready[slot] == u.  The last wave to finish a block
  // (counted in done[slot] against the number of waves that need it) refills the slot with block
  // u + NS and publishes it after its loads have landed: right away if it is about to wait for a
  // block itself, otherwise after its next block of work, running at raised wave priority
  // until then.  Every wait is bounded.
  int pending = -1;       // stream entry this wave loaded and has not published yet
  bool stalled = false;
  // The wave reads 64 list entries at a time and jumps straight to the blocks its tokens chose.
  for (int ubase = 0; ubase < n_union && !stalled; ubase += 64) {
    const MaskT chunk = ubase + lane < n_union ? umask[ubase + lane] : MaskT{0};
    const int chunk_blk = ubase + lane < n_union ? static_cast<int>(ublk[ubase + lane]) : 0;
    unsigned long long todo = __ballot(((chunk >> (TPW * w)) & ((MaskT{1} << TPW) - 1u)) != 0u);
   while (todo != 0ull) {
    const int bit = __builtin_ctzll(todo);
    todo &= todo - 1ull;
    const int u = ubase + bit;
    MaskT ent = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(chunk), bit));
    if constexpr (sizeof(MaskT) == 8)
      ent |= static_cast<MaskT>(static_cast<uint32_t>(
                 __builtin_amdgcn_readlane(static_cast<int>(chunk >> 32), bit))) << 32;
    const uint32_t wm = static_cast<uint32_t>((ent >> (TPW * w)) & ((MaskT{1} << TPW) - 1u));
    const int slot = u % NS;
    if (lds_peek(&ready[slot]) != u) {
      if (pending >= 0) {
        wait_vmcnt<0>();
        lds_store(&ready[pending % NS], pending);
        pending = -1;
        __builtin_amdgcn_s_setprio(0);
      }
      int spins = 0;
      while (lds_peek(&ready[slot]) != u) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) { stalled = true; break; }
      }
      if (stalled) break;
    }
    asm volatile("" ::: "memory");
    const int key0 = __builtin_amdgcn_readlane(chunk_blk, bit) * 64;
    const uint32_t slot_off = static_cast<uint32_t>(slot) * (2 * MAT);
    const lds_bf16x8* Kp = (const lds_bf16x8*)(uintptr_t)(k_lane + slot_off);
    const uint32_t vaddr = v_lane + slot_off;
#pragma unroll
    for (int tt = 0; tt < CG; ++tt) {
      const uint32_t gm = (wm >> (TPC * tt)) & ((1u << TPC) - 1u);   // the group's tokens
      if (gm == 0u) continue;
      const int pos = pos0 + TPW * w + TPC * tt + ct;                 // this lane's token
      const int pos_lo = pos0 + TPW * w + TPC * tt;                   // the group's first token
      if constexpr (BWD) {
        // S^T = K Q^T and dP^T = V dO^T in the same key order; P = exp(S*scale - lse) from the
        // forward's statistics (no running max), dS = P (dP - delta), dQ += dS K.
        f32x4 sa[2][2], pa4[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int tp = 0; tp < 2; ++tp) {
            sa[s][tp] = f32x4{0.f, 0.f, 0.f, 0.f};
            pa4[s][tp] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        bf16x8 ka[KS][2][2], va[KS][2][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
              ka[ks][s][tp] = Kp[((2 * s + tp) * KS + ks) * 64];
              va[ks][s][tp] =
                  *(const lds_bf16x8*)(uintptr_t)(kofs[ks] + slot_off + MAT + (32 * s + 4 * tp) * 2 * D);
            }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
              sa[s][tp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks][s][tp], qf[tt][ks], sa[s][tp], 0, 0, 0);
              pa4[s][tp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ks][s][tp], dof[tt][ks], pa4[s][tp], 0, 0, 0);
            }
        sched_reads_ahead<KS, 8, 1>();
        const int lim = (key0 + 63 > pos || key0 + 64 > kv_len) ? min(pos, kv_len - 1) - key0 : 63;
        const float nl = -lse2[tt];
        const float dd = dl[tt];
        float dsv[2][2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float p = 32 * s + 8 * q4 + 4 * tp + i > lim
                                  ? 0.f
                                  : __builtin_amdgcn_exp2f(fmaf(sa[s][tp][i], qscale, nl));
              dsv[s][tp][i] = p * (pa4[s][tp][i] - dd);
            }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x2 d01 = __builtin_convertvector((f32x2){dsv[s][0][0], dsv[s][0][1]}, bf16x2);
          const bf16x2 d23 = __builtin_convertvector((f32x2){dsv[s][0][2], dsv[s][0][3]}, bf16x2);
          const bf16x2 d45 = __builtin_convertvector((f32x2){dsv[s][1][0], dsv[s][1][1]}, bf16x2);
          const bf16x2 d67 = __builtin_convertvector((f32x2){dsv[s][1][2], dsv[s][1][3]}, bf16x2);
          const bf16x2 dp[4] = {d01, d23, d45, d67};
          const bf16x8 dsa = __builtin_bit_cast(bf16x8, dp);
          uint64_t kt[NT][2];   // read x = NT h + n lands in kt[x / 2][x % 2]
          read_v_half<NT>(vaddr + 512u * (2 * NT * s), kt);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const uint64_t both[2] = {kt[n / 2][n % 2], kt[NT / 2 + n / 2][n % 2]};
            o[tt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dsa, __builtin_bit_cast(bf16x8, both),
                                                               o[tt][n], 0, 0, 0);
          }
        }
        continue;
      }
      // S^T tiles: tile (s, tp) row r' -> key 32s + 8(r'/4) + 4tp + (r'%4); the lane then
      // holds keys 32s + 8*q4 + 4*tp + i for head c16 (raw, unscaled dot products).
      // the four (s, tp) accumulator chains advance together, one k-step at a time
      f32x4 acc4[2][2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) acc4[s][tp] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 kf[KS][2][2];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int tp = 0; tp < 2; ++tp)
            kf[ks][s][tp] = *(const lds_bf16x8*)(uintptr_t)(kofs[ks] + slot_off + (32 * s + 4 * tp) * 2 * D);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int tp = 0; tp < 2; ++tp)
            acc4[s][tp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks][s][tp], qf[tt][ks], acc4[s][tp], 0, 0, 0);
      // instruction order: the first two k-steps' reads, then the MFMAs, each followed by a
      // read two k-steps ahead (left to itself the scheduler waits for nearly every read right
      // before its MFMA)
      sched_reads_ahead<KS, 4, 2>();
      float sv[2][2][4];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[s][tp][i] = acc4[s][tp][i];
      // keys past the query or the sequence end (only in the query's own block or the tail),
      // with a window, keys before it, and every key of a stacked token that did not choose
      // the block
      const bool partial = TPC > 1 && gm != (1u << TPC) - 1u;
      if (partial || key0 + 63 > pos_lo || key0 + 64 > kv_len || (WIN && key0 <= pos - g.window)) {
        int lim = min(pos, kv_len - 1) - key0;
        if (TPC > 1 && !((gm >> ct) & 1u)) lim = -1;
        const int lo = WIN ? pos - g.window + 1 - key0 : 0;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int kk = 32 * s + 8 * q4 + 4 * tp + i;
              if (kk > lim || kk < lo) sv[s][tp][i] = -INFINITY;
            }
      }
      float mx = sv[0][0][0];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[s][tp][i]);
      mx *= qscale;
      // lazy rescaling: the running max moves only when some head's block max exceeds it by
      // more than kLazy (probabilities then stay below 2^kLazy), decided for the whole wave
      if (__ballot(mx > m_run[tt] + kLazy) != 0ull) {
        float bm = fmaxf(mx, __shfl_xor(mx, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float m_new = fmaxf(m_run[tt], bm);
        // a stacked column with no key yet keeps -inf (its sums are still 0)
        const float alpha = (TPC > 1 && m_new == -INFINITY) ? 1.f
                                                             : __builtin_amdgcn_exp2f(m_run[tt] - m_new);
        l_run[tt] *= alpha;
        m_run[tt] = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a_i = __shfl(alpha, 4 * q4 + i);
#pragma unroll
          for (int n = 0; n < NT; ++n) o[tt][n][i] *= a_i;
        }
      }
      const float mneg = (TPC > 1 && m_run[tt] == -INFINITY) ? 0.f : -m_run[tt];
      float psum = 0.f;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sv[s][tp][i], qscale, mneg));
            sv[s][tp][i] = p;
            psum += p;
          }
      l_run[tt] += psum;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // P operand: head c16, keys 32s + 8*q4 + 0..7
        const bf16x2 p01 = __builtin_convertvector((f32x2){sv[s][0][0], sv[s][0][1]}, bf16x2);
        const bf16x2 p23 = __builtin_convertvector((f32x2){sv[s][0][2], sv[s][0][3]}, bf16x2);
        const bf16x2 p45 = __builtin_convertvector((f32x2){sv[s][1][0], sv[s][1][1]}, bf16x2);
        const bf16x2 p67 = __builtin_convertvector((f32x2){sv[s][1][2], sv[s][1][3]}, bf16x2);
        const bf16x2 pp[4] = {p01, p23, p45, p67};
        const bf16x8 pa = __builtin_bit_cast(bf16x8, pp);
        uint64_t vt[NT][2];
        read_v_half<NT>(vaddr + 512u * (2 * NT * s), vt);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const uint64_t both[2] = {vt[n][0], vt[n][1]};
          const bf16x8 vb = __builtin_bit_cast(bf16x8, both);
          o[tt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[tt][n], 0, 0, 0);
        }
      }
    }
    wait_lgkm0();
    if (pending >= 0) {                      // publish the block loaded one step earlier
      wait_vmcnt<0>();
      lds_store(&ready[pending % NS], pending);
      pending = -1;
      __builtin_amdgcn_s_setprio(0);
    }
    // done accounting; the last of the block's waves refills the slot
    const MaskT mk = ent;
    const int needers = count_wave_groups<TPW, NW>(mk);
    int old = 0;
    if (lane == 0) old = atomicAdd(&done[slot], 1);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old + 1 == needers) {
      if (lane == 0) lds_store(&done[slot], 0);
      if (u + NS < n_union) {
        // other waves wait for this refill: the wave issues it and runs at raised priority
        // until it has published it (its SIMD's other wave yields issue slots meanwhile)
        __builtin_amdgcn_s_setprio(2);
        produce(u + NS, slot, 0, 1);
        pending = u + NS;
      }
    }
   }
  }
  if (pending >= 0) {
    wait_vmcnt<0>();
    lds_store(&ready[pending % NS], pending);
  }

  if constexpr (BWD) {
    // dQ = scale * sum_j dS_j k_j, fp32, same [row, head, dim] layout as q
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int tw = TPW * w + tt;
      if (tw >= nq) continue;
      const float f = stalled ? __builtin_nanf("") : g.scale;
      const size_t orow = static_cast<size_t>(row0 + tw) * Hq + kvh * G;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * q4 + i;
        if (h < G) {
          float* dp = dq + (orow + h) * D;
#pragma unroll
          for (int n = 0; n < NT; ++n) dp[16 * n + c16] = o[tt][n][i] * f;
        }
      }
    }
    return;
  }

  // ---- epilogue: combine the 4 lanes' partial sums, normalise and store.  Accumulator row h
  // (4 q4 + i) is column h of S: token TPW*w + TPC*tt + h / G, head h % G.
#pragma unroll
  for (int tt = 0; tt < CG; ++tt) {
    if (TPW * w + TPC * tt >= nq) continue;
    float l = l_run[tt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (stalled) l = __builtin_nanf("");     // never expected: flags the row instead of hanging
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * q4 + i;
      const int tw = TPW * w + TPC * tt + (TPC == 1 ? 0 : h / G);
      const int hh = TPC == 1 ? h : h % G;
      const float inv = 1.f / __shfl(l, h);
      if (hh < G && tw < nq) {
        uint16_t* op = out + ((static_cast<size_t>(row0 + tw) * Hq + kvh * G + hh) * D);
#pragma unroll
        for (int n = 0; n < NT; ++n) op[16 * n + c16] = f32_to_bf16(o[tt][n][i] * inv);
      }
    }
    const int tl = TPW * w + TPC * tt + ct;
    if (lse != nullptr && q4 == 0 && hd < G && tl < nq)
      lse[static_cast<size_t>(row0 + tl) * Hq + kvh * G + hd] = (m_run[tt] + log2f(l)) * kLn2;
  }
}

}  // namespace

bool attn_tile_supported(const Geom& g, int dtype, const SeqTable& t) {
  return dtype == INFLLM2_BF16 && g.B == 64 && (g.d == 64 || g.d == 128) &&
         (g.G == 8 || g.G == 16) && bound_blocks(t, 64) <= kMaxUnion;
}

// Compute units of the current device, looked up once per device.  The cache is shared by every
// calling thread: relaxed atomics (racing first calls store the same value).
int device_cus() {
  static std::atomic<int> cached[64];                 // static storage: starts at 0
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Tiles are scheduled in rounds of one workgroup per compute unit, so that the workgroups
// sharing an XCD start together on neighbouring tiles and walk the same KV blocks at the same
// time (their L2 then serves each block to all of them): a round is 8 groups of gs = CUs / 8
// consecutive tiles (locate_group).  A launch holds kRoundsPerLaunch rounds: the next round's
// workgroups take the compute units the current round's tail frees (measured at 128K: 29.6 ms
// with one round per launch, 29.2 / 29.0 / 29.2 with 2 / 3 / 4, 30.2 with every round in one
// launch, whose workgroups drift apart and stop sharing staged blocks in the XCD's L2).  The
// forward runs tiles of kTF8 rows at G = 8 (a wave's 4 tokens fill two 16-column MFMA groups;
// kTF8S rows, 8 tokens in four groups, at head_dim 64, whose accumulators are half as large) and
// of kTF rows at G = 16 (a round of 24-token tiles takes ~1.4 times as long as one of 16-token
// tiles for 1.5 times the tokens; with the next round filling a round's tail, 24 also beats 16 on
// a 16K-token chunk of few rounds: 5.28 against 5.37 ms).
static int group_tiles() { return std::max(1, device_cus() / 8); }

// Bound on the number of tile groups of a launch (tiles of `rows` rows, gs tiles per group): at
// most ceil(ceil(max_q_len / rows) / gs) per (sequence, KV head), and, since a sequence of len
// rows has fewer than len / (rows gs) + 1 groups, at most ceil(q_rows / (rows gs)) + n in all.
static int bound_groups(const SeqTable& t, int rows, int gs, int hkv) {
  const long long per_seq = ((static_cast<long long>(t.max_q_len) + rows - 1) / rows + gs - 1) / gs;
  const long long a = static_cast<long long>(t.n) * per_seq;
  const long long span = static_cast<long long>(rows) * gs;
  const long long c = (static_cast<long long>(t.q_rows) + span - 1) / span + t.n;
  return static_cast<int>((a < c ? a : c) * hkv);
}

static int attn_tile_rows(const Geom& g) {
  if (g.G == 8) return g.d == 64 ? kTF8S : kTF8;
  return kTF;
}

hipError_t launch_attn_tile(const Geom& g, const SeqTable& t, const void* q, const void* k,
                            const void* v, const int32_t* idx, void* out, float* lse,
                            hipStream_t stream) {
  const int TF = attn_tile_rows(g);
  const int gs = group_tiles();
  const int n_groups = bound_groups(t, TF, gs, g.Hkv);   // a bound: the kernel finds the groups
  if (n_groups == 0) return hipSuccess;
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(out);
  for (int base = 0; base < n_groups; base += 8 * kRoundsPerLaunch) {
    const int grid = 8 * kRoundsPerLaunch * gs;
#define INFLLM2_TILE_CASE(DD, GG, NS, TFF)                                                    \
  if (g.d == DD && g.G == GG && TF == TFF) {                                                  \
    hipLaunchKernelGGL((attn_tile<DD, GG, NS, kWavesF, TFF / kWavesF, false, false, true>),   \
                       dim3(grid),                                                            \
                       dim3(64 * kWavesF), 0, stream, g, t, qq, kk, vv, idx, oo, lse, base,  \
                       nullptr, nullptr, nullptr, nullptr);                                   \
    const hipError_t e = hipGetLastError();                                                   \
    if (e != hipSuccess) return e;                                                            \
    continue;                                                                                 \
  }
    INFLLM2_TILE_CASE(128, 16, 4, kTF)
    INFLLM2_TILE_CASE(128, 8, 4, kTF8)
    INFLLM2_TILE_CASE(64, 16, 8, kTF)
    INFLLM2_TILE_CASE(64, 8, 8, kTF8S)
#undef INFLLM2_TILE_CASE
    return hipErrorInvalidValue;
  }
  return hipSuccess;
}

// Gradient of the queries (tiles of kT rows): dout is the
// upstream gradient of out, lse the forward's natural-log statistics and delta[row, head] =
// dout . out.  Writes dq (fp32, [row, Hq, d]) for every row of every sequence.
hipError_t launch_attn_tile_dq(const Geom& g, const SeqTable& t, const void* q, const void* k,
                               const void* v, const int32_t* idx, const void* dout,
                               const float* lse, const float* delta, float* dq,
                               hipStream_t stream) {
  const int gs = group_tiles();
  const int n_groups = bound_groups(t, kT, gs, g.Hkv);
  if (n_groups == 0) return hipSuccess;
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  const uint16_t* dd = static_cast<const uint16_t*>(dout);
  for (int base = 0; base < n_groups; base += 8 * kRoundsPerLaunch) {
    const int grid = 8 * kRoundsPerLaunch * gs;
#define INFLLM2_DQ_CASE(DD, GG, NS)                                                           \
  if (g.d == DD && g.G == GG) {                                                               \
    hipLaunchKernelGGL((attn_tile<DD, GG, NS, kWaves, kT / kWaves, true, false, true>),       \
                       dim3(grid),                                                            \
                       dim3(64 * kWaves), 0, stream, g, t, qq, kk, vv, idx, nullptr, nullptr, \
                       base, dd, lse, delta, dq);                                             \
    const hipError_t e = hipGetLastError();                                                   \
    if (e != hipSuccess) return e;                                                            \
    continue;                                                                                 \
  }
    INFLLM2_DQ_CASE(128, 16, 4)
    INFLLM2_DQ_CASE(128, 8, 4)
    INFLLM2_DQ_CASE(64, 16, 8)
    INFLLM2_DQ_CASE(64, 8, 8)
#undef INFLLM2_DQ_CASE
    return hipErrorInvalidValue;
  }
  return hipSuccess;
}

hipError_t launch_attn_tile_window(const Geom& g, const SeqTable& t, const void* q,
                                   const void* k, const void* v, void* out, float* lse,
                                   hipStream_t stream) {
  const int gs = group_tiles();
  const int n_groups = bound_groups(t, kTW, gs, g.Hkv);
  if (n_groups == 0) return hipSuccess;
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(out);
  for (int base = 0; base < n_groups; base += 8 * kRoundsPerLaunch) {
    const int grid = 8 * kRoundsPerLaunch * gs;
#define INFLLM2_WIN_CASE(DD, GG, NS)                                                          \
  if (g.d == DD && g.G == GG) {                                                               \
    hipLaunchKernelGGL((attn_tile<DD, GG, NS, kWaves, kTW / kWaves, false, true>), dim3(grid), \
                       dim3(64 * kWaves), 0, stream, g, t, qq, kk, vv, nullptr, oo, lse,      \
                       base, nullptr, nullptr, nullptr, nullptr);                             \
    const hipError_t e = hipGetLastError();                                                   \
    if (e != hipSuccess) return e;                                                            \
    continue;                                                                                 \
  }
    INFLLM2_WIN_CASE(128, 16, 4)
    INFLLM2_WIN_CASE(128, 8, 4)
    INFLLM2_WIN_CASE(64, 16, 8)
    INFLLM2_WIN_CASE(64, 8, 8)
#undef INFLLM2_WIN_CASE
    return hipErrorInvalidValue;
  }
  return hipSuccess;
}

}  // namespace infllm2
