// Output-error loss of each grid point:  L_k = || dW_k X^T ||_F^2  (fp16 MFMA, fp32
// accumulation, fp64 per-tile partials), and the argmin.  One kernel, three modes:
//   direct     C = dW_k X^T, each 256 x 256 tile squared and summed in registers;
//   G loss     the same L_k as sum_r dW_r G dW_r^T with G = X^T X: C = G' dW_k^T over the
//              block upper triangle of G, epilogue sum dW (C + dW diag(G));
//   G build    G itself, from X^T, as 256 x 256 tiles of its upper block triangle.
//
// Pages: "AWQ" scholia-log notes §1.1 (output error Delta Y = Delta W X) and §4.1
// (argmin of the squared Frobenius norm over the scale family); ewbang.com GPTQ与AWQ
// §3 二 (objective ||WX - Q(W s)(X/s)|| with a grid search over alpha in [0, 1]).
//
// dW_k is fp16 [M][K] and X is fp16 [N][K]: both operands are K-contiguous, so C = dW X^T
// is a "TN" product whose tiles stream straight from HBM (so are G' [K][K] and X^T [K][N]
// in the G modes).  No product is stored except G in the build mode.
//
// Design for CDNA4 (gfx950, wave64, 160 KiB LDS per CU, 64-bank LDS):
//   block = 8 waves (2 x 4), tile 256 dW rows x 256 tokens, wave sub-tile 128 x 64 =
//   4 x 2 MFMA 32x32x16 f16 blocks (128 fp32 accumulators per lane, two waves per SIMD).
//   K streams through LDS 64 channels per stage in a ring of NS stages.  Operands move
//   global -> LDS with the gfx950 buffer_load ... lds DMA (no register staging): lane l
//   of a wave-DMA lands at LDS byte 16 l of a 1 KiB block, and out-of-range offsets
//   (rows past the matrix, channels past in_features) arrive as zeros.  A stage buffer
//   is refilled right after the barrier that follows the last fragment read from it,
//   with explicit s_waitcnt accounting (the number of DMAs in flight is constant).
//   Rows of a stage are 128 bytes; the 16-byte chunk index is XOR-swizzled with
//   (row & 7) ^ ((row >> 3) & 1), which keeps every 16 consecutive rows on 16 distinct
//   16-byte bank groups modulo 256 bytes, so fragment reads are conflict-free.
//   Fragments ping-pong between two register sets so the LDS reads of step k+1 overlap
//   the MFMAs of step k.
//   MFMA operand layout (32x32x16 f16): lane l supplies row (l mod 32) and channels
//   8*(l div 32) .. +7 of the 16-channel slice for A, and the same for B with tokens
//   in place of rows.  The loss only needs the sum of squares of the output tile, so the
//   accumulator layout never has to be decoded.
//   Block-to-tile map: hardware hands block b to XCD (b mod 8); blocks are renumbered so
//   each XCD walks a contiguous range of tiles, ordered in bands of 4 tile-rows (8
//   tile-row pairs in the G form), which keeps the panels its 32 CUs share resident in
//   that XCD's L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "awq_act.h"
#include "awq_internal.h"

// Stage geometry, overridable for sweeps; the defaults (64 channels per stage, 2 stages,
// 2 x 4 waves) are the fastest measured on MI355X.
#ifndef LOSS_BK
#define LOSS_BK 64
#endif
#ifndef LOSS_NS
#define LOSS_NS 2
#endif
#ifndef LOSS_WM
#define LOSS_WM 2
#endif
#ifndef LOSS_WN
#define LOSS_WN 4
#endif
// G form: each pass runs its k-tiles from the last one down to its diagonal block (1), so
// that the tile's own dW block is in LDS when the pass ends, or upwards (0).
#ifndef LOSS_GRAM_REV
#define LOSS_GRAM_REV 1
#endif
// Keep each k-step's fragment reads for the next k-step ahead of the current MFMAs (1), or
// leave their placement to the compiler (0).  The default eight-wave tiling runs the same
// either way (two waves per SIMD hide the reads); four waves of 128 x 128 need 1, where the
// compiler otherwise issues a k-step's reads right before its own MFMAs.
#ifndef LOSS_SB
#define LOSS_SB 0
#endif
// Raised wave priority around the fragment reads and refill DMAs (1) or none (0).
#ifndef LOSS_PRIO
#define LOSS_PRIO 1
#endif

namespace awq {

namespace {

constexpr int BM = kLossBM, BN = kLossBN;
constexpr int kBandM = 4;  // tile-rows per raster band (direct form)
constexpr int kBandG = 8;  // tile-row pairs per raster band (G form; same-device sweep: 8 over 4 and 2)

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

typedef int int32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource (gfx9 layout): 48-bit base, stride 0, byte range, 32-bit data
// format.  Accesses at offsets >= num_bytes return zero.
__device__ __forceinline__ int32x4 make_rsrc(const void* base, unsigned num_bytes) {
  const unsigned long long b = (unsigned long long)base;
  int32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)(b & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)((b >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)num_bytes);
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (int)(unsigned)(size_t)(const __attribute__((address_space(3))) void*)p);
}

// One wave-level 16-byte-per-lane DMA from global memory into LDS: lane l's 16 bytes at
// buffer offset voff + soff land at LDS byte lds + 16 l.  Issued as inline assembly so
// that the compiler's automatic waits do not drain the DMA queue before unrelated LDS
// reads; every wait for these transfers is the explicit s_waitcnt at the barriers.
// The instruction writes no VGPR (its data goes to LDS), so no register of the asm is
// overwritten after the statement.
__device__ __forceinline__ void dma16(const int32x4& rsrc, unsigned lds, unsigned voff,
                                      unsigned soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}

// s_waitcnt immediate for gfx9: vmcnt(vm) with expcnt/lgkmcnt: lgkmcnt(0), expcnt(7).
template <int VM>
struct WaitVmLgkm {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  static constexpr int value = (VM & 0xF) | ((VM >> 4) << 14) | (7 << 4);
};

// Tile geometry: a K slice of BK channels per stage, NS stages, WM x WN waves.
template <int BK_, int NS_, int WM_, int WN_>
struct Stage {
  static constexpr int BK = BK_;
  static constexpr int NS = NS_;
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int MI = BM / WM / 32;                     // 32-row MFMA blocks per wave
  static constexpr int NI = BN / WN / 32;                     // 32-token MFMA blocks per wave
  static constexpr int CPR = BK / 8;                          // 16-byte chunks per row
  static constexpr int ROWS_PER_DMA = 64 / CPR;               // rows one wave-DMA fills
  static constexpr int DMA_A = BM * BK * 2 / 1024 / WAVES;    // DMAs per wave for A
  static constexpr int DMA_B = BN * BK * 2 / 1024 / WAVES;
  static constexpr int PER_STAGE = DMA_A + DMA_B;             // vmcnt units per stage
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int BYTES = (BM + BN) * BK * 2;
  static constexpr int KSTEPS = BK / 16;
  static_assert(DMA_A >= 1 && DMA_B >= 1, "each wave issues at least one DMA per operand");
  // XOR swizzle of the 16-byte chunk index within a row.  A fragment read has the 32
  // lanes of a half-wave on 32 consecutive rows at the same logical chunk; the swizzle
  // spreads every 16 consecutive rows over 16 distinct 16-byte slots modulo 256 bytes
  // (and every 8 over 8 slots modulo 128 bytes), so neither a 64-bank nor a 32-bank
  // LDS sees a conflict.  128-byte rows: (row & 7) ^ ((row >> 3) & 1);
  // 64-byte rows: ((row >> 1) & 3) ^ ((row >> 3) & 1).  Both depend on row & 15 only.
  __device__ static int swz(int row) {
    return CPR == 8 ? ((row & 7) ^ ((row >> 3) & 1)) : (((row >> 1) & 3) ^ ((row >> 3) & 1));
  }
};

// MODE kModeDirect: C = dW_k X^T (X fp16 [N][K]) and the tile's sum of squares.
// MODE kModeGramLoss (GRAM below): C = G' dW_k^T with G' 2^-gexp fp16 [K][K] passed as X
// (N = K): the A side of the tile is channels (rows of G'), the B side rows of dW_k.  G' is
// G with its BM x BM blocks above the diagonal doubled, those below it zero and its
// diagonal zero, so tile row tm needs k from tm BM on only; inside each diagonal block the
// same holds at half size, so the tile's channels BM / 2 .. BM - 1 need k from
// tm BM + BM / 2 on (their waves skip the first half block).  The tile's sum over its
// positions (c, r) of dW_k[r][c] (C[c][r] + dW_k[r][c] gdiag[c]), with gdiag = diag(G)
// 2^-gexp in fp32, times 2^gexp, is the tile's share of sum_r dW_r G dW_r^T.  With channels
// on the A side, the four consecutive C rows a lane holds are four consecutive channels of
// one dW row, so the epilogue reads its dW in 8-byte pieces (from the tile's dW block,
// staged in LDS).
// MODE kModeGramBuild (BUILD below): G = X^T X itself from Xt = X^T (fp16 [K][ld], tokens
// contiguous, passed as X): the A and B sides are both channels, the reduction runs over
// the tokens [s kchunk, min(N, (s + 1) kchunk)) of split s (passed as the grid point), and
// only tiles tm <= tn of G's upper block triangle are formed.  Each split's fp32 tile goes
// to gout = partial tiles [split][pair][BM][BN] and its largest |entry| to
// tmax[split][pair].
constexpr int kModeDirect = 0, kModeGramLoss = 1, kModeGramBuild = 2;
template <class S, int MODE>
__global__ __launch_bounds__(S::THREADS) void k_loss_gemm(
    const uint16_t* __restrict__ dW, const uint16_t* __restrict__ X,
    const float* __restrict__ gdiag, int M, int N, int K, int ld, int kchunk, int tiles_m,
    int tiles_n, int nb, const int32_t* __restrict__ gexp, double* __restrict__ partials,
    float* __restrict__ gout, float* __restrict__ tmax) {
  constexpr bool GRAM = MODE == kModeGramLoss;
  constexpr bool BUILD = MODE == kModeGramBuild;
  // One LDS array per pipeline stage: distinct objects let the compiler see that a DMA
  // into one stage never aliases fragment reads from another, so it does not drain the
  // DMA queue before every LDS read.
  __shared__ __attribute__((aligned(1024))) uint8_t sm0[S::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sm1[S::NS > 1 ? S::BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sm2[S::NS > 2 ? S::BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sm3[S::NS > 3 ? S::BYTES : 16];
  // REV (the G form in reverse k order) fills the whole 160 KiB: two stages and a spare
  // buffer for the tile's upper 64 dW channels; its reduction slots and diag(G) staging
  // then live in stage memory that is free when they are used.
  constexpr bool REV = GRAM && LOSS_GRAM_REV;
  __shared__ __attribute__((aligned(1024))) uint8_t smx[REV ? (BN * S::BK * 2) : 16];
  __shared__ double red_a[S::WAVES];
  __shared__ float redf[S::WAVES];
  __shared__ __attribute__((aligned(16))) float gds_a[GRAM && !REV ? BM : 4];
  static_assert(!REV || (S::NS == 2 && S::BK == 64 && 2 * S::BYTES + BN * S::BK * 2 == 163840),
                "the reverse G form fills the LDS exactly");
  static_assert(S::NS >= 2 && S::NS <= 4, "2..4 stages");

  const int tid = threadIdx.x;
  // wave index as a scalar (uniform) value, so LDS bases derived from it live in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave / S::WN;
  const int wn = wave % S::WN;

  // ---- block -> (grid point, tile row, tile column), XCD-contiguous ----------------
  // GRAM: tile row tm covers k from tm BM on, so a block takes the pair of tile rows tm
  // and tiles_m - 1 - tm (tiles_m + 1 blocks of G' between them): equal work per block.
  // BUILD: grid point = token split, and a block's tile is the rem-th pair tm <= tn of
  // the upper block triangle in row-major order.
  // BUILD: the splits are dispatched in order (all blocks of split 0 first), and within a
  // split each XCD takes a contiguous run of pairs; XCDs take blocks round-robin, so every
  // XCD starts on the longer splits and gets an even share of each split.
  const int tm_count = GRAM ? (tiles_m + 1) / 2 : tiles_m;
  const int per_alpha = BUILD ? tiles_m * (tiles_m + 1) / 2 : tm_count * tiles_n;
  const int b = blockIdx.x;
  const int split_b = BUILD ? b / per_alpha : 0;
  const int bb = b - split_b * per_alpha;
  const int total = BUILD ? per_alpha : nb * per_alpha;
  const int xcd = bb & 7;
  const int local = bb >> 3;
  const int q = total >> 3, r = total & 7;
  const int logical = (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  const int kk_alpha = BUILD ? split_b : logical / per_alpha;
  const int rem = BUILD ? logical : logical - kk_alpha * per_alpha;
  int tm, tn;
  if constexpr (BUILD) {
    int t = 0, left = rem;
    while (left >= tiles_m - t) {
      left -= tiles_m - t;
      ++t;
    }
    tm = t;
    tn = t + left;
  } else {
    constexpr int BMB = GRAM ? kBandG : kBandM;
    const int band = rem / (BMB * tiles_n);
    const int first_m = band * BMB;
    const int band_rows = min(BMB, tm_count - first_m);
    const int in_band = rem - band * BMB * tiles_n;
    tm = first_m + in_band % band_rows;
    tn = in_band / band_rows;
  }
  // reduction length KR of this block and row stride LD of both operands
  const int k_first = BUILD ? kk_alpha * kchunk : 0;
  const int KR = BUILD ? min(kchunk, N - k_first) : K;
  const int LD = BUILD ? ld : K;

  const uint16_t* B = BUILD  ? X + (size_t)tn * BN * LD + k_first
                      : GRAM ? dW + (size_t)kk_alpha * M * K + (size_t)tn * BN * K
                             : X + (size_t)tn * BN * K;
  const int rows_b = BUILD ? min(BN, K - tn * BN) : GRAM ? min(BN, M - tn * BN) : min(BN, N - tn * BN);

  // ---- DMA through buffer resources.  Lane l of a wave-level buffer_load ... lds fills
  //      LDS bytes [16 l, 16 l + 16) of a 1 KiB block: row l / CPR of the block,
  //      physical chunk l % CPR, which holds logical chunk (l % CPR) ^ swz(row) (swz
  //      depends only on the lane for these blocks).  The per-lane byte offset is fixed;
  //      the block index and the K position go into the scalar offset.  Rows past the
  //      end of the tile and channels past in_features fall outside the resource's
  //      range, and the hardware writes zeros for them.
  // A wave-DMA block covers ROWS_PER_DMA (8 or 16) rows starting at a multiple of that
  // count, so row & 15 is (block parity) * 8 + lane / CPR when blocks hold 8 rows.
  const int dma_row_in = lane / S::CPR;
  const int dma_lchunk_even = (lane % S::CPR) ^ S::swz(dma_row_in);
  const int dma_lchunk_odd = (lane % S::CPR) ^ S::swz(dma_row_in + (S::ROWS_PER_DMA == 8 ? 8 : 0));
  int32x4 rsrc_a;  // set per tile row (part) below
  const int32x4 rsrc_b = make_rsrc(B, (unsigned)rows_b * (unsigned)LD * 2u);
  static_assert(S::DMA_A % 2 == 0 && S::DMA_B % 2 == 0, "block parity follows j");
  const unsigned row_a = (unsigned)(wave * S::DMA_A * S::ROWS_PER_DMA + dma_row_in);
  const unsigned row_b = (unsigned)(wave * S::DMA_B * S::ROWS_PER_DMA + dma_row_in);
  const unsigned vo_a0 = (row_a * (unsigned)LD + dma_lchunk_even * 8) * 2u;
  const unsigned vo_a1 = (row_a * (unsigned)LD + dma_lchunk_odd * 8) * 2u;
  const unsigned vo_b0 = (row_b * (unsigned)LD + dma_lchunk_even * 8) * 2u;
  const unsigned vo_b1 = (row_b * (unsigned)LD + dma_lchunk_odd * 8) * 2u;
  const unsigned dma_row_stride = (unsigned)S::ROWS_PER_DMA * (unsigned)LD * 2u;  // bytes per j
  constexpr unsigned kOutOfRange = 0x80000000u;

  auto stage_ptr = [&](auto st) -> uint8_t* {
    constexpr int ST = decltype(st)::value;
    if constexpr (ST == 0) return sm0;
    else if constexpr (ST == 1) return sm1;
    else if constexpr (ST == 2) return sm2;
    else return sm3;
  };

  // LDS byte addresses of the stage buffers (uniform, computed once).
  const unsigned lds_stage[4] = {lds_addr(sm0), lds_addr(sm1), lds_addr(sm2), lds_addr(sm3)};
  const unsigned lds_spare = REV ? lds_addr(smx) : 0u;

  // k-tiles rounded up to a multiple of NS: the padding tiles lie past the reduction
  // length, read as zeros and add nothing, and the NS-unrolled loop below then has a
  // single exit.
  const int nk = ((KR + S::BK * S::NS - 1) / (S::BK * S::NS)) * S::NS;
  // GRAM: k-tiles kt0 .. nk - 1 (kt0 a multiple of NS since BM / BK is); set per part
  static_assert(!GRAM || (BM / S::BK) % S::NS == 0, "the diagonal block starts on a whole pipeline step");
  int kt0 = 0, nkt = nk;

  // loop tile i -> k-tile kt0 + i (REV: nk - 1 - i); past the end: zeros, or (REV) nothing,
  // since the stages then hold the tile's dW block for the epilogue
  // REV, the last two refills (loop tiles nkt - 2 and nkt - 1, k-tiles kt0 + 1 and kt0, in
  // stages 0 and 1): the A rows BM / 2 .. BM - 1 of those k-tiles are zero in G' (the lower-left
  // half of the diagonal block), so the waves that would load them (wave >= WAVES / 2) load
  // dW channels kt0 + 2 of the tile instead, rows 0 .. 127 into stage 0 and rows 128 .. 255
  // into stage 1 (A-region row 128 + (r mod 128)), and with the first of them every wave
  // loads its rows of channels kt0 + 3 into the spare buffer.
  const unsigned epi_shift = (unsigned)(BM / 2) * (unsigned)LD * 2u;  // 128 dW rows, bytes
  auto dma_stage = [&](auto st, int i) {
    constexpr int ST = decltype(st)::value;
    if constexpr (REV) {
      if (i >= nkt) return;
    }
    const int k0 = (i < nkt ? (REV ? nk - 1 - i : kt0 + i) : nk) * S::BK;
    const unsigned la = lds_stage[ST] + (unsigned)(wave * S::DMA_A) * 1024u;
    const unsigned lb = lds_stage[ST] + (unsigned)S::A_BYTES + (unsigned)(wave * S::DMA_B) * 1024u;
    const bool k_ok0 = k0 + dma_lchunk_even * 8 < KR;
    const bool k_ok1 = k0 + dma_lchunk_odd * 8 < KR;
    const unsigned va0 = k_ok0 ? vo_a0 : kOutOfRange, va1 = k_ok1 ? vo_a1 : kOutOfRange;
    const unsigned vb0 = k_ok0 ? vo_b0 : kOutOfRange, vb1 = k_ok1 ? vo_b1 : kOutOfRange;
    const unsigned kbytes = (unsigned)k0 * 2u;
    bool epi = false;
    if constexpr (REV) epi = nkt >= 4 && i == nkt - 2 + ST && wave >= S::WAVES / 2;
    if (!epi) {
#pragma unroll
      for (int j = 0; j < S::DMA_A; ++j)
        dma16(rsrc_a, la + j * 1024u, (j & 1) ? va1 : va0, kbytes + j * dma_row_stride);
    } else {
      // dW rows (wave - WAVES/2) 32 + ... of channels kt0 + 2 into the A-region rows 128 + ...
      const int ke = (kt0 + 2) * S::BK;
      const bool e0 = ke + dma_lchunk_even * 8 < KR, e1 = ke + dma_lchunk_odd * 8 < KR;
      const unsigned sh = ST == 0 ? epi_shift : 0u;
      const unsigned ve0 = e0 ? vo_b0 - sh : kOutOfRange, ve1 = e1 ? vo_b1 - sh : kOutOfRange;
#pragma unroll
      for (int j = 0; j < S::DMA_A; ++j)
        dma16(rsrc_b, la + j * 1024u, (j & 1) ? ve1 : ve0, (unsigned)ke * 2u + j * dma_row_stride);
    }
#pragma unroll
    for (int j = 0; j < S::DMA_B; ++j)
      dma16(rsrc_b, lb + j * 1024u, (j & 1) ? vb1 : vb0, kbytes + j * dma_row_stride);
    if constexpr (REV && ST == 0) {
      if (nkt >= 4 && i == nkt - 2) {  // channels kt0 + 3 of every row into the spare buffer
        const int ks3 = (kt0 + 3) * S::BK;
        const bool s0 = ks3 + dma_lchunk_even * 8 < KR, s1 = ks3 + dma_lchunk_odd * 8 < KR;
        const unsigned vs0 = s0 ? vo_b0 : kOutOfRange, vs1 = s1 ? vo_b1 : kOutOfRange;
        const unsigned ls = lds_spare + (unsigned)(wave * S::DMA_B) * 1024u;
#pragma unroll
        for (int j = 0; j < S::DMA_B; ++j)
          dma16(rsrc_b, ls + j * 1024u, (j & 1) ? vs1 : vs0, (unsigned)ks3 * 2u + j * dma_row_stride);
      }
    }
  };

  // ---- fragment reads: MFMA 32x32x16 f16 operand = row (l mod 32), channels
  //      8*(l div 32) .. +7 of the 16-channel step, for A (dW rows) and B (tokens).
  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  const int frag_swz = S::swz(frag_row);
  const int a_off = (wm * S::MI * 32 + frag_row) * S::BK * 2;
  const int b_off = S::A_BYTES + (wn * S::NI * 32 + frag_row) * S::BK * 2;

  struct Frag {
    half8 a[S::MI], b[S::NI];
  };
  // The two waves of a SIMD alternate between fragment reads and MFMAs; a wave issuing
  // its reads runs at raised priority, so the next step's operands are requested before
  // the other wave's MFMAs take the issue slots (same-device A/B of the 20-alpha search,
  // three rounds: 1.696 against 1.727 ms; priority around the MFMAs instead: 1.698).
  auto load_frag = [&](auto st, int ks, Frag& f) {
    if constexpr (LOSS_PRIO) __builtin_amdgcn_s_setprio(1);
    const uint8_t* base = stage_ptr(st);
    const int chunk = ((2 * ks + frag_half) ^ frag_swz) * 16;
#pragma unroll
    for (int mi = 0; mi < S::MI; ++mi)
      f.a[mi] = *(const half8*)(base + a_off + mi * 32 * S::BK * 2 + chunk);
#pragma unroll
    for (int ni = 0; ni < S::NI; ++ni)
      f.b[ni] = *(const half8*)(base + b_off + ni * 32 * S::BK * 2 + chunk);
    if constexpr (LOSS_PRIO) __builtin_amdgcn_s_setprio(0);
  };

  floatx16 acc[S::MI][S::NI];

  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int mi = 0; mi < S::MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < S::NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0);
  };

  // ---- pipeline: NS stages in flight; a stage buffer is refilled right after the
  //      barrier that follows the last fragment read from it.  DMAs are issued for
  //      every stage slot (past the end of K they read zeros into a slot nobody reads),
  //      so the number of DMAs in flight, hence the vmcnt to wait for, is constant.
  //      The K loop is unrolled by NS so that every access names its stage array.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1 % S::NS>;
  using I2 = std::integral_constant<int, 2 % S::NS>;
  using I3 = std::integral_constant<int, 3 % S::NS>;
  static_assert(S::KSTEPS % 2 == 0, "even number of 16-channel steps per stage");
  Frag f0, f1;

  // one k-tile held in stage ST (k-tile index kt)
  auto step = [&](auto st, int kt) {
    constexpr int ST = decltype(st)::value;
    using NEXT = std::integral_constant<int, (ST + 1) % S::NS>;
    auto sb = [&]() {
      if constexpr (LOSS_SB) __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int ks = 0; ks + 2 < S::KSTEPS; ks += 2) {
      load_frag(st, ks + 1, f1);
      sb();
      mma(f0);
      load_frag(st, ks + 2, f0);
      sb();
      mma(f1);
    }
    load_frag(st, S::KSTEPS - 1, f1);
    sb();
    mma(f0);
    // stage kt+1 has landed (own DMAs) and this wave's reads of stage kt are done
    __builtin_amdgcn_s_waitcnt(WaitVmLgkm<(S::NS - 2) * S::PER_STAGE>::value);
    __builtin_amdgcn_s_barrier();
    // the refill DMAs, too, go out at raised priority (same-device A/B, three rounds: loss
    // product 1.339 against 1.370 ms)
    if constexpr (LOSS_PRIO) __builtin_amdgcn_s_setprio(1);
    dma_stage(st, kt + S::NS);
    if constexpr (LOSS_PRIO) __builtin_amdgcn_s_setprio(0);
    load_frag(NEXT{}, 0, f0);  // after the last k-tile this reads a slot nobody uses
    if constexpr (LOSS_SB) __builtin_amdgcn_sched_barrier(0);
    mma(f1);
  };

  // GRAM: a part's first BM / 2 channels of k are the first half of its diagonal block,
  // where G' is zero for the tile's channels BM / 2 .. BM - 1 (its lower-left half block).
  // The waves holding those channels (wm == 1) only keep the pipeline going there: the
  // barrier, their share of the refill DMAs and the next stage's first fragments.
  static_assert(!GRAM || (S::WM == 2 && (BM / 2) / S::BK == S::NS),
                "the idle pass is one NS-stage iteration over half a diagonal block");
  auto step_idle = [&](auto st, int kt) {
    constexpr int ST = decltype(st)::value;
    using NEXT = std::integral_constant<int, (ST + 1) % S::NS>;
    __builtin_amdgcn_s_waitcnt(WaitVmLgkm<(S::NS - 2) * S::PER_STAGE>::value);
    __builtin_amdgcn_s_barrier();
    if constexpr (LOSS_PRIO) __builtin_amdgcn_s_setprio(1);
    dma_stage(st, kt + S::NS);
    if constexpr (LOSS_PRIO) __builtin_amdgcn_s_setprio(0);
    load_frag(NEXT{}, 0, f0);
  };
  const bool idle_first = GRAM && wm == 1;

  double ssum = 0.0;
  float gmx = 0.0f;     // BUILD: largest |entry| of the tile
  float gd_pre = 0.0f;  // GRAM: this thread's entry of the tile's diag(G)
  // One pass per tile row of the block (two for a GRAM pair).  Between passes no barrier
  // is needed: every wave's DMAs of the next pass go to its own LDS blocks after its own
  // vmcnt(0), and other waves have finished their fragment reads of the last real stage
  // at the final barrier of the previous pass (the read after it only loads a register
  // set nobody uses).
  const int nparts = (GRAM && tiles_m - 1 - tm != tm) ? 2 : 1;
  for (int part = 0; part < nparts; ++part) {
  // the blocks of a pair set that share a dW panel stream the same k-tile of it at the same
  // time during their long row, so they share its reads in L2: in forward k order the short
  // row (tiles_m - 1 - tm) comes first, in reverse order (REV) the long row (tm), both rows
  // ending at their diagonal blocks
  const int tmc = ((part == 0) == (nparts == 2)) != REV ? tiles_m - 1 - tm : tm;
  {
    const uint16_t* A = BUILD  ? X + (size_t)tmc * BM * LD + k_first
                        : GRAM ? X + (size_t)tmc * BM * K
                               : dW + (size_t)kk_alpha * M * K + (size_t)tmc * BM * K;
    const int rows_a = BUILD ? min(BM, K - tmc * BM) : GRAM ? min(BM, N - tmc * BM) : min(BM, M - tmc * BM);
    rsrc_a = make_rsrc(A, (unsigned)rows_a * (unsigned)LD * 2u);
    if constexpr (GRAM) {
      kt0 = min(tmc * (BM / S::BK), nk);
      nkt = nk - kt0;
      // diag(G) of the tile's channels, in flight during the pass (0 past in_features)
      const int c = tmc * BM + tid;
      gd_pre = (tid < BM && c < N) ? gdiag[c] : 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < S::MI; ++i)
#pragma unroll
    for (int j = 0; j < S::NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  dma_stage(I0{}, 0);
  if constexpr (S::NS > 1) dma_stage(I1{}, 1);
  if constexpr (S::NS > 2) dma_stage(I2{}, 2);
  if constexpr (S::NS > 3) dma_stage(I3{}, 3);
  __builtin_amdgcn_s_waitcnt(WaitVmLgkm<(S::NS - 1) * S::PER_STAGE>::value);
  __builtin_amdgcn_s_barrier();

  // Fragments ping-pong between two register sets; KSTEPS is even, so a stage always
  // starts with its first k-step in f0 and ends having loaded the next stage's first
  // k-step into f0 as well.
  if (nk > 0) load_frag(I0{}, 0, f0);

  int kt_begin = 0, kt_end = nkt;
  if constexpr (GRAM && !REV) {
    if (idle_first && nkt > 0) {  // wave-uniform
      step_idle(I0{}, 0);
      if constexpr (S::NS > 1) step_idle(I1{}, 1);
      if constexpr (S::NS > 2) step_idle(I2{}, 2);
      if constexpr (S::NS > 3) step_idle(I3{}, 3);
      kt_begin = S::NS;
    }
  }
  if constexpr (REV) {
    if (idle_first) kt_end = nkt - S::NS;  // the half block comes last (nkt >= 2, even)
  }
  for (int kt = kt_begin; kt < kt_end; kt += S::NS) {
    step(I0{}, kt);
    if constexpr (S::NS > 1) step(I1{}, kt + 1);
    if constexpr (S::NS > 2) step(I2{}, kt + 2);
    if constexpr (S::NS > 3) step(I3{}, kt + 3);
  }
  if constexpr (REV) {
    if (idle_first) {
      step_idle(I0{}, nkt - 2);
      step_idle(I1{}, nkt - 1);
    }
  }
  __builtin_amdgcn_s_waitcnt(WaitVmLgkm<0>::value);  // no LDS write may outlive the block

  // ---- epilogue: sum of squares of the 256 x 256 output tile (GRAM: sum of
  //      dW (C + dW gdiag) at the output positions; BUILD: the tile itself); element e
  //      of a 32x32 block is row 8 (e / 4) + 4 (l / 32) + (e mod 4), column l mod 32 ----
  if constexpr (BUILD) {
    // the split's partial of the tile, row-major within the tile (a row-contiguous
    // 128-byte run per half-wave and e); entries past in_features are not written
    const int pair = rem;
    float* dst = gout + ((size_t)kk_alpha * per_alpha + pair) * (BM * BN);
#pragma unroll
    for (int mi = 0; mi < S::MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < S::NI; ++ni) {
        const int bl = wn * S::NI * 32 + ni * 32 + (lane & 31);
        const int al0 = wm * S::MI * 32 + mi * 32 + 4 * (lane >> 5);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int al = al0 + 8 * (e >> 2) + (e & 3);
          if (tm * BM + al < K && tn * BN + bl < K) {
            const float v = acc[mi][ni][e];
            dst[(size_t)al * BN + bl] = v;
            gmx = (fabsf(v) > gmx || v != v) ? fabsf(v) : gmx;
          }
        }
      }
  } else if constexpr (REV) {
    // The tile's own dW block is in LDS already: channels 0..63 of the tile in stage 1's B
    // half (k-tile kt0), 64..127 in stage 0's B half (kt0 + 1), 128..191 in the A regions'
    // rows 128..255 (dW rows 0..127 in stage 0, 128..255 in stage 1), 192..255 in the spare
    // buffer; each region has 128-byte rows with the stages' chunk swizzle.  diag(G) of the
    // tile goes to stage 0's A rows 0..3, free once every wave has passed the last barrier.
    float* gds = (float*)sm0;
    __syncthreads();
    if (tid < BM) gds[tid] = gd_pre;
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < S::MI; ++mi) {
      const int cl = wm * S::MI * 32 + mi * 32 + 4 * (lane >> 5);  // channel within the tile
      const int q = cl >> 6;                                        // 64-channel slice
#pragma unroll
      for (int ni = 0; ni < S::NI; ++ni) {
        const int rl = wn * S::NI * 32 + ni * 32 + (lane & 31);   // row within the tile
        const uint8_t* rowp;
        if (q == 0)      rowp = sm1 + S::A_BYTES + rl * (S::BK * 2);
        else if (q == 1) rowp = sm0 + S::A_BYTES + rl * (S::BK * 2);
        else if (q == 2) rowp = (rl < BM / 2 ? sm0 : sm1) + ((rl & (BM / 2 - 1)) + BM / 2) * (S::BK * 2);
        else             rowp = smx + rl * (S::BK * 2);
        const int sw = S::swz(rl);
        float tsum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = cl + 8 * j;                                   // first of 4 channels
          const floatx4 g4 = *(const floatx4*)(gds + c);
          u32x2 w2 = *(const u32x2*)(rowp + ((((c & 63) >> 3) ^ sw) * 16) + 8 * (lane >> 5));
          if (tmc * BM + c >= N) w2 = u32x2{0u, 0u};                  // past in_features
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const unsigned w = w2[qq >> 1];
            const float d = (float)__builtin_bit_cast(
                _Float16, (uint16_t)(qq & 1 ? w >> 16 : w & 0xffffu));
            tsum = fmaf(d, fmaf(d, g4[qq], acc[mi][ni][4 * j + qq]), tsum);
          }
        }
        ssum += (double)tsum;
      }
    }
    __syncthreads();  // the next tile row's DMAs reuse the stage buffers
  } else if constexpr (GRAM) {
    // The tile's own dW block (its 256 rows x its 256 channels) is staged through the
    // stage buffers, free now: every wave's DMAs have landed (vmcnt(0) above, then the
    // barrier), and every fragment read of them finished before the loop's last barrier.
    // Rows 0..127 go to sm0, 128..255 to sm1, 512 bytes each, the 16-byte chunk q of row r
    // at chunk position q ^ (r & 31): one wave-DMA moves two whole rows (coalesced), and the
    // output-layout reads below (32 rows, one chunk column) spread over the banks.  Rows
    // past out_features lie past the tile's resource and read zeros; chunks past
    // in_features take the out-of-range offset (K is a multiple of 8, so a chunk is wholly
    // inside or outside).
    static_assert(S::NS >= 2 && S::BYTES >= (BM / 2) * BN * 2, "two stage buffers hold the block");
    static_assert(BM == 256 && BN == 256 && (BN / S::WAVES) % 2 == 0, "epilogue staging geometry");
    constexpr int kRowsPerWave = BN / S::WAVES;  // tile rows each wave stages, two per DMA
    __syncthreads();
    {
      // rsrc_b is this tile's rows of dW_k (at most 256 K 2 bytes from row tn BN)
      const int half = lane >> 5, pos = lane & 31;
#pragma unroll
      for (int i = 0; i < kRowsPerWave / 2; ++i) {
        const int rl = wave * kRowsPerWave + 2 * i + half;  // row within the tile (uniform pair)
        const int q = pos ^ (rl & 31);                // logical chunk held at position pos
        const int c = tmc * BM + 8 * q;
        const unsigned voff = c < N ? ((unsigned)rl * (unsigned)K + (unsigned)c) * 2u : kOutOfRange;
        const int rpair = wave * kRowsPerWave + 2 * i;  // first row of this DMA (uniform)
        const unsigned lds = (rpair < 128 ? lds_stage[0] + (unsigned)rpair * 512u
                                          : lds_stage[1] + (unsigned)(rpair - 128) * 512u);
        dma16(rsrc_b, lds, voff, 0u);
      }
    }
    float* gds = gds_a;
    if (tid < BM) gds[tid] = gd_pre;
    __builtin_amdgcn_s_waitcnt(WaitVmLgkm<0>::value);
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < S::MI; ++mi) {
      const int cl = wm * S::MI * 32 + mi * 32 + 4 * (lane >> 5);  // channel within the tile
#pragma unroll
      for (int ni = 0; ni < S::NI; ++ni) {
        const int rl = wn * S::NI * 32 + ni * 32 + (lane & 31);   // row within the tile
        const uint8_t* rowp = (rl < 128 ? sm0 + rl * 512 : sm1 + (rl - 128) * 512);
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const floatx4 g4 = *(const floatx4*)(gds + cl + 8 * j);
          const int q = (wm * S::MI * 32 + mi * 32 + 8 * j) / 8;   // logical chunk
          const u32x2 w2 = *(const u32x2*)(rowp + ((q ^ (rl & 31)) * 16) + 8 * (lane >> 5));
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const unsigned w = w2[qq >> 1];
            const float d = (float)__builtin_bit_cast(
                _Float16, (uint16_t)(qq & 1 ? w >> 16 : w & 0xffffu));
            t = fmaf(d, fmaf(d, g4[qq], acc[mi][ni][4 * j + qq]), t);
          }
        }
        ssum += (double)t;
      }
    }
    __syncthreads();  // the next tile row's DMAs reuse the stage buffers
  } else {
#pragma unroll
    for (int mi = 0; mi < S::MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < S::NI; ++ni) {
        float t = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) t += acc[mi][ni][e] * acc[mi][ni][e];
        ssum += (double)t;
        __builtin_amdgcn_sched_barrier(0);  // one 32x32 block at a time: low VGPR pressure
      }
  }
  }  // part
  if constexpr (BUILD) {
    // the largest |entry| of the split's partial tile (NaN if any entry is NaN)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float o = __shfl_xor(gmx, off);
      gmx = (o > gmx || o != o) ? o : gmx;
    }
    if (lane == 0) redf[wave] = gmx;
    __syncthreads();
    if (tid == 0) {
      float m = redf[0];
#pragma unroll
      for (int w = 1; w < S::WAVES; ++w) m = (redf[w] > m || redf[w] != redf[w]) ? redf[w] : m;
      tmax[(size_t)kk_alpha * per_alpha + rem] = m;
    }
    return;
  }
  double* red = REV ? (double*)sm1 : red_a;  // REV: stage 1 is free after the last epilogue
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ssum += __shfl_xor(ssum, off);
  if (lane == 0) red[wave] = ssum;
  __syncthreads();
  if (tid == 0) {
    double t = red[0];
#pragma unroll
    for (int w = 1; w < S::WAVES; ++w) t += red[w];
    if constexpr (GRAM) t = ldexp(t, gexp[0]);
    double* part_k = partials + (size_t)kk_alpha * tiles_m * tiles_n;
    part_k[(size_t)tm * tiles_n + tn] = t;
    if (nparts == 2) part_k[(size_t)(tiles_m - 1 - tm) * tiles_n + tn] = 0.0;
  }
}

using LossStage = Stage<LOSS_BK, LOSS_NS, LOSS_WM, LOSS_WN>;
// The direct product and the Gram build run sixteen waves of 128 x 32 (four a SIMD, 64
// accumulators a wave): their epilogues fit the 128 registers that leaves, and the extra
// waves hide more of the fragment reads.  The G form's loss epilogue does not fit them
// and keeps eight waves.
#ifndef LOSS_WN_WIDE
#define LOSS_WN_WIDE 8
#endif
using LossStageWide = Stage<LOSS_BK, LOSS_NS, LOSS_WM, LOSS_WN_WIDE>;

// Per-alpha loss = fixed-order fp64 sum of its tile partials (wave w handles alphas
// w, w + 16, ...: lane-strided sums, then a butterfly in a fixed order), then the argmin
// over finite losses (first index on ties) and the chosen scale vector.
constexpr int kSelectThreads = 1024;

__global__ __launch_bounds__(kSelectThreads) void k_reduce_select(
    const double* __restrict__ partials, int n_alpha, int tiles, const float* __restrict__ s_table,
    int K, double* __restrict__ losses, int32_t* __restrict__ best_out,
    int32_t* __restrict__ status_out, float* __restrict__ s_out) {
  __shared__ double lsh[kMaxAlpha];
  __shared__ int best_sh;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  for (int k = wave; k < n_alpha; k += kSelectThreads / 64) {
    double acc = 0.0;
    for (int i = lane; i < tiles; i += 64) acc += partials[(size_t)k * tiles + i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) {
      lsh[k] = acc;
      losses[k] = acc;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int best = -1;
    double bl = 0.0;
    for (int k = 0; k < n_alpha; ++k) {
      const double l = lsh[k];
      if (isfinite(l) && (best < 0 || l < bl)) {
        best = k;
        bl = l;
      }
    }
    best_sh = best;
    best_out[0] = best;
    if (status_out) status_out[0] = best < 0 ? AWQ_W_NONFINITE : AWQ_OK;
  }
  __syncthreads();
  const int best = best_sh;
  for (int i = tid; i < K; i += kSelectThreads)
    s_out[i] = best >= 0 ? s_table[(size_t)best * K + i] : 1.0f;
}

}  // namespace

hipError_t launch_loss_gemm(const uint16_t* dW, const uint16_t* X, int M, int N, int K, int nb,
                            double* partials, hipStream_t stream) {
  if (M <= 0 || N <= 0 || nb <= 0) return hipSuccess;
  const int tm = (int)loss_tiles_m(M), tn = (int)loss_tiles_n(N);
  const long long blocks = (long long)nb * tm * tn;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_loss_gemm<LossStageWide, kModeDirect>), dim3((unsigned)blocks),
                     dim3(LossStageWide::THREADS), 0, stream, dW, X, nullptr, M, N, K, K, 0, tm, tn,
                     nb, nullptr, partials, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_loss_gemm_gram(const uint16_t* dW, const uint16_t* Gh, const float* gdiag,
                                 const int32_t* gexp, int M, int K, int nb, double* partials,
                                 hipStream_t stream) {
  static_assert(kLossBM == kLossBN, "the G form uses square tiles (G's blocks)");
  if (M <= 0 || K <= 0 || nb <= 0) return hipSuccess;
  // tile rows over channels (rows of G'), tile columns over rows of dW; a block takes a
  // pair of tile rows
  const int tm = (int)loss_tiles_m(K), tn = (int)loss_tiles_n(M);
  const long long blocks = (long long)nb * ((tm + 1) / 2) * tn;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_loss_gemm<LossStage, kModeGramLoss>), dim3((unsigned)blocks),
                     dim3(LossStage::THREADS), 0, stream, dW, Gh, gdiag, M, K, K, K, 0, tm, tn,
                     nb, gexp, partials, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_gram_build(const uint16_t* Xt, int N, int ld, int K, int kchunk, int splits,
                             float* out, float* tmax, hipStream_t stream) {
  if (K <= 0 || N <= 0 || splits <= 0) return hipSuccess;
  if (kchunk % 8 != 0 || ld % 8 != 0) return hipErrorInvalidValue;
  const int T = (int)loss_tiles_m(K);
  const long long blocks = (long long)splits * T * (T + 1) / 2;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_loss_gemm<LossStageWide, kModeGramBuild>), dim3((unsigned)blocks),
                     dim3(LossStageWide::THREADS), 0, stream, nullptr, Xt, nullptr, 0, N, K, ld,
                     kchunk, T, T, splits, nullptr, nullptr, out, tmax);
  return hipGetLastError();
}

hipError_t launch_reduce_select(const double* partials, int n_alpha, int tiles,
                                const float* s_table, int K, double* losses, int32_t* best,
                                int32_t* status, float* s_out, hipStream_t stream) {
  hipLaunchKernelGGL(k_reduce_select, dim3(1), dim3(kSelectThreads), 0, stream, partials, n_alpha,
                     tiles, s_table, K, losses, best, status, s_out);
  return hipGetLastError();
}

}  // namespace awq
