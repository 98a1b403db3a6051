// Block-scaled FP8 GEMM with FP32 promotion every 128 K, dense and grouped.
//
// Method: why-be.co.kr as_center post 57820, promotion passage (at the end of
// every N_C interval the partial result leaves the matrix unit, is multiplied
// by the scaling factors and added into FP32 registers on the general ALUs);
// pkd.ac.th webboard post 78017, increased-precision accumulation passage
// (N_C = 128); the-good.kr free board post 2169793 (per-group scaling along K,
// dequantized on the general ALUs).
//
// MI355X mapping.  One v_mfma_f32_16x16x128_f8f6f4 consumes exactly one
// 128-wide K chunk of a 16x16 output block, so each chunk's partial P_g is a
// single MFMA started from zero; the promotion acc = fma(P_g, s_a*s_w, acc) is
// four VALU FMAs per MFMA.  The product is formed transposed (C^T = W A^T:
// MFMA rows are weight rows, MFMA columns are activation rows), so a lane's
// four results of a block share one activation row and one multiplier, and
// are four consecutive outputs (one 16-byte store).  Inside a wave the blocks
// are software pipelined: block k's partial is folded by the VALU while the
// matrix core runs the next MFMAs (the role the pages give to two alternating
// warpgroups on Hopper).
//
// Each wave owns 64 (48 in the grouped 160- and 192-row tiles) activation rows
// and 128 weight rows inside one 128-row weight block, so s_w is one
// wave-uniform scalar per chunk, and the row scales of a row of waves are one
// 256-byte LDS slot per chunk.  Operands move HBM/L2 -> LDS with 16-byte
// direct-to-LDS buffer loads (no VGPR staging) through a ring of STAGES K
// chunks with one barrier per chunk; the loads of the chunks ahead are spread
// over the MFMA sequence, and the next chunk's fragments are read
// into registers before the current chunk's last MFMAs, so the matrix core
// does not drain at chunk boundaries.  LDS rows are 128 bytes (one K chunk)
// with the 16-byte column index XOR-swizzled per row so fragment reads are
// bank-conflict free.  The dense kernel's two-stage ring is backed by an L2
// prefetch several chunks ahead, split between the tiles that share a band
// of A or W rows in one XCD's L2.
//
// The same tile serves more configurations (GemmCfg flags): the
// weight-gradient GEMM, whose weight-side operand carries 1x128 row-group
// scales like the activations (W_ROWSCALE: the multiplier differs per output
// element); BF16 operands without scales (OP = kOpBf16: the reference of the
// FP8 path, accumulating in the matrix core); the precise mode (OP =
// kOpWide16: the E4M3 codes, unchanged in LDS, are widened exactly to FP16 in
// registers and each chunk's partial is formed by FP16 MFMAs, whose FP32
// accumulation has no narrow truncation step); power-of-two scales applied by
// the matrix core as E8M0 operand scales (OP = kOpFp8Mx, the pages' "MMA with
// group scaling" wish: the partial comes out scaled and the promotion is an
// add); BF16 activations quantized on their way into LDS (A_CAST, see
// ACaster); and the grouped MoE kernel's row-count buckets (persistent
// workgroups, see grouped_gemm_kernel).

#include <type_traits>

#include "gemm_common.hpp"
#include "quant_rules.hpp"

namespace fp8q {

// OP_: the operands and the matrix-core instruction.
//   kOpFp8   : E4M3 codes; one 16x16x128 FP8 MFMA forms a block's chunk
//              partial from zero.
//   kOpBf16  : BF16 operands (the reference GEMM of the same kernel family):
//              a 128-byte stage row then holds 64 K values, each 16x16 block
//              takes two chained 16x16x32 BF16 MFMAs per chunk, accumulating
//              in the matrix core (its BF16 path accumulates to FP32
//              accuracy), and there are no scales.
//   kOpWide16: E4M3 codes staged exactly as for kOpFp8, widened to FP16 in
//              registers after the fragment read (exact: every E4M3 value is
//              an FP16 value), and a block's chunk partial is four chained
//              16x16x32 FP16 MFMAs from zero (the precise mode: the FP8
//              MFMA truncates products inside 8-product groups, the FP16 one
//              accumulates its exact products to FP32 accuracy).
//   kOpFp8Mx : E4M3 codes with power-of-two scales, which the matrix core
//              applies itself: the block-scaled FP8 MFMA takes each group
//              scale as an E8M0 byte (the lanes that supply a row's operand
//              supply its byte), so a chunk partial comes out already
//              scaled, from zero, and the promotion is a plain FP32 add.
// W_ROWSCALE_: the weight-side operand carries 1x128 row-group scales
// ([K/128][N], like the activations) instead of 128x128 block scales: the
// weight-gradient GEMM, whose operands dY^T and X^T are both grouped along
// the tokens.  The multiplier then differs per output element.
// A_CAST_: 0 = the activation codes and row scales are loaded as they are;
// 1 (FP32 scales) or 2 (power-of-two scales) = the activations arrive as BF16
// and are quantized on their way into LDS (ACaster).
constexpr int kOpFp8 = 0, kOpBf16 = 1, kOpWide16 = 2, kOpFp8Mx = 3;
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_, int ROWS_ = BM_,
          int PF_ = 0, int OP_ = kOpFp8, int W_ROWSCALE_ = 0, int A_CAST_ = 0>
struct GemmCfg {
  static constexpr bool OP_BF16 = OP_ == kOpBf16;
  static constexpr bool WIDE16 = OP_ == kOpWide16;
  static constexpr bool MX = OP_ == kOpFp8Mx;
  static constexpr bool W_ROWSCALE = W_ROWSCALE_ != 0;
  static constexpr bool A_CAST = A_CAST_ != 0;
  static constexpr int CAST_MODE = A_CAST ? A_CAST_ - 1 : 0;
  // MFMAs per 16x16 block per chunk
  static constexpr int SUB = OP_BF16 ? 2 : WIDE16 ? 4 : 1;
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int BK = 128;                    // bytes of K per stage row and chunk
  static constexpr int WAVES_M = WAVES_M_;
  static constexpr int WAVES_N = WAVES_N_;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = NWAVES * 64;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int MB = WM / 16;                // MFMA row blocks per wave
  static constexpr int NB = WN / 16;                // MFMA column blocks per wave
  static constexpr int ROWS = ROWS_;                // A rows staged per chunk (<= BM)
  static constexpr int A_BYTES = ROWS * BK;
  static constexpr int B_BYTES = BN * BK;
  static constexpr int SA_BYTES = OP_BF16 ? 0 : WAVES_M * 256;  // 64 row scales per row of waves
  // the tile's weight-row scales: 4 slots of 64 (rows past BN loaded, unused)
  static constexpr int SB_BYTES = W_ROWSCALE ? 4 * 256 : 0;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
  static constexpr int STAGES = STAGES_;
  static constexpr int PF_LOADS = PF_;    // L2 prefetch loads per wave per chunk (0 or 1)
  static constexpr int PF_BYTES = PF_LOADS > 0 ? NWAVES * 256 : 0;  // their LDS landing slots
  static constexpr int LDS_BYTES = STAGE * STAGES + PF_BYTES;
  static constexpr int A_BLK = A_CAST ? 0 : A_BYTES / 1024;  // 1 KiB load instructions for A
  static constexpr int OP_BLK = A_BLK + B_BYTES / 1024;
  static constexpr int PER_WAVE = (OP_BLK + NWAVES - 1) / NWAVES;  // operand loads per wave
  static constexpr int PAD = PER_WAVE * NWAVES - OP_BLK;  // repeated A loads that even them out
  static constexpr int LOADS =
      PER_WAVE + (OP_BF16 || A_CAST ? 0 : 1) + (W_ROWSCALE ? 1 : 0);  // + scales
  static constexpr int CAST_ROUNDS = A_CAST ? (ROWS + 63) / 64 : 0;  // 64 rows per round
  static_assert(WM % 16 == 0 && WM <= 64, "a wave's rows fit one 256-byte scale slot");
  static_assert(W_ROWSCALE || 128 % WN == 0,
                "a wave's weight rows lie in one 128-row weight block (block-scaled weights)");
  // Staged rows: whole 1 KiB loads.  When they stop inside a wave (160 rows
  // in 48-row waves), that wave's fragment reads past them fall inside the
  // stage and feed only rows past the expert's end, which are not stored.
  static_assert(ROWS % 32 == 0 && ROWS <= BM, "staged rows fill whole loads within the tile");
  static_assert(PAD <= A_BLK, "the padding loads repeat A loads");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 2 && STAGES <= 6, "ring depth");
  static_assert(PF_LOADS == 0 || (PF_LOADS == 1 && NWAVES >= 2 && ROWS == 256 && BN == 256),
                "the prefetch share is laid out for 256 x 256 tiles");
  static_assert(LOADS * (STAGES - 1) + PF_LOADS * (STAGES - 1) < 64, "vmcnt range");
  static_assert(!W_ROWSCALE || (!OP_BF16 && NWAVES == 8 && WAVES_N == 2 && BN <= 256),
                "row-scaled weights: 8 waves, each loading 64 of up to 256 row scales");
  static_assert(!A_CAST || (OP_ == kOpFp8 && !W_ROWSCALE && PF_LOADS == 0 && THREADS == 512 &&
                            A_CAST_ <= 2 && CAST_ROUNDS <= 4),
                "activation cast: 512 lanes, 8 per row, FP8 block-scaled weights");
  static_assert(OP_ >= kOpFp8 && OP_ <= kOpFp8Mx, "operand mode");
  static_assert(!MX || (!W_ROWSCALE && !A_CAST), "matrix-core scales: block-scaled dense GEMM");
};

// Dense configuration: 256 x 256 tiles, 8 waves (two per SIMD, so one wave's
// promotion FMAs overlap the other's MFMAs), 2 stages (132 KiB of LDS) and an
// L2 prefetch kPfDist chunks ahead (a ring of 2 stages leaves the loads of a
// chunk less than one chunk's compute time to arrive from HBM).
using DenseCfg = GemmCfg<256, 256, 4, 2, 2, 256, 1>;
// The BF16 GEMM: the same tile, waves, ring and prefetch.
using DenseBf16Cfg = GemmCfg<256, 256, 4, 2, 2, 256, 1, kOpBf16>;
// The precise mode: the same tile, waves, ring and prefetch, FP16 MFMAs on
// the widened codes.
using DenseWideCfg = GemmCfg<256, 256, 4, 2, 2, 256, 1, kOpWide16>;
// Power-of-two scales applied by the matrix core: the same tile, waves, ring
// and prefetch.
using DenseMxCfg = GemmCfg<256, 256, 4, 2, 2, 256, 1, kOpFp8Mx>;
// The weight-gradient GEMM: the dense tile with row-scaled weights.
using RowScaledCfg = GemmCfg<256, 256, 4, 2, 2, 256, 1, kOpFp8, 1>;
using RowScaledWideCfg = GemmCfg<256, 256, 4, 2, 2, 256, 1, kOpWide16, 1>;
// The same with 224-row weight tiles (waves of 64 x 112; row-scaled weights
// have no 128-row blocks to respect), for shapes where they fill the CUs'
// rounds better: 4096 x 7168 outputs make 448 tiles of 256 x 256 (a second
// round 3/4 full on 256 CUs) but 512 of 256 x 224 (two full rounds of
// 7/8-size tiles).  No L2 prefetch (its share is laid out for 256 x 256).
using RowScaled224Cfg = GemmCfg<256, 224, 4, 2, 2, 256, 0, kOpFp8, 1>;
// BF16 activations quantized inside the GEMM (scale mode MODE): the dense
// tile without the L2 prefetch, whose A lines would be BF16 rows.
template <int MODE>
using DenseCastCfg = GemmCfg<256, 256, 4, 2, 2, 256, 0, kOpFp8, 0, 1 + MODE>;
// Grouped configurations: 256-row tiles cover an expert's tokens (decode
// batches hold at most 256) so each expert's weights stream once, and 256
// weight rows per tile (8 waves of 64 x 128, as in the dense tile) so each
// expert's activation rows are re-read from L2 by N/256 tiles rather than
// N/128 (at 128 weight rows the activation reads outweighed the weight
// stream in large tiles and held the weight stream below the copy rate).
// Only the tile's live rows are staged (64, 128, 160, 192 or 256), and the
// LDS this frees deepens the ring: 3 stages up to 160 rows, 2 above.  A
// 2-stage ring streams the weights markedly slower than a 3-stage one once
// the activation rows share the loads, so 160 rows (most experts of a
// 256-expert top-8 routing of 4096 tokens hold 103..157) get a bucket of
// their own: the largest that still fits 3 stages in 160 KiB.
constexpr int kGroupedBN = 256;
// 160- and 192-row tiles hold experts of 129..192 rows: their waves take 48
// rows each, so for up to 144 rows the fourth row of waves has none and
// skips its MFMAs (64-row waves would run three full waves for 129 rows).
// CAST: 0, or 1 + the scale mode of activations quantized inside the GEMM
// (the same LDS ring: the cast writes the codes where the loads would).
// OP: kOpFp8, or kOpWide16 for the precise mode (no cast).
template <int ROWS, int S, int CAST = 0, int OP = kOpFp8>
using GroupedCfg =
    GemmCfg<(ROWS == 160 || ROWS == 192 ? 192 : 256), kGroupedBN, 4, 2, S, ROWS, 0, OP, 0, CAST>;
constexpr int kS64 = 3, kS128 = 3, kS160 = 3, kS192 = 2, kS256 = 2;

// Main-loop schedule constants (measured on the 4096 x 4096 x 7168 shape;
// the result is insensitive to them within +-2%):
//   kDma0, kDmaStep  head load d of the next chunk goes out after MFMA
//                    kDma0 + d * kDmaStep;
//   kPromoteLag      a block's partial is promoted this many MFMAs after it
//                    was issued, when the matrix core has surely written it;
//   kBPrefetch       weight fragments are read this many row blocks ahead;
//   kBarLead         the chunk barrier sits this many MFMAs before the
//                    chunk's last row block.
//   kPfDist          the L2 prefetch issued while chunk g is computed
//                    touches chunk g + kPfDist.
constexpr int kPfDist = 6;
constexpr int kDma0 = 1;
constexpr int kDmaStep = 2;
constexpr int kPromoteLag = 2;
constexpr int kBPrefetch = 1;
constexpr int kBarLead = 2;

// Direct-to-LDS loads of one K chunk (A rows, W rows, row scales).  The
// operand tiles are cut into 1 KiB load instructions (8 rows of 128 B):
// instructions 0 .. A_BLK-1 carry A rows, the next ones W rows, and load d
// of wave w is instruction d*NWAVES + w, so every wave issues its share of
// the A rows first and then its share of the W rows (waves that issued only
// A or only W rows streamed the weights of the grouped tiles 1-2% slower);
// then comes the 256-byte slot of its row of waves' row scales (both waves
// of a row write the same values there): Cfg::LOADS instructions per wave
// per chunk.  When the operand loads do not split evenly over the waves, the
// last PAD instructions repeat the first A loads (same bytes to the same LDS
// place).  Lane
// i of an instruction lands at LDS byte 16*i, i.e. row i/8, physical column
// i%8, and so fetches logical column swz(row, i%8).  Rows past the valid range
// are clamped to the last valid row (their results are never stored).
//
// Addresses are buffer offsets: a scalar resource per operand based at the
// tile's first row, a per-lane 32-bit offset fixed for the whole tile, and the
// chunk's K offset as the scalar soffset, so issuing a load costs no VALU.
template <class Cfg>
struct ChunkLoader {
  __amdgpu_buffer_rsrc_t ra, rw, rs, rsb;
  uint32_t voff[Cfg::PER_WAVE];
  uint32_t voff_s;
  uint32_t voff_sb;   // this lane's weight-row scale (row-scaled weights)
  int64_t sb_stride;  // bytes between consecutive chunks' weight-row scales
  uint32_t voff_pf;  // this lane's L2 prefetch line (first byte of its K chunk)
  bool pf_a;         // the wave prefetches A rows (else W rows)
  int64_t s_stride;  // bytes between consecutive chunks' row scales
  int wave, wave_m;

  // Operand block of load instruction m (the padding repeats A blocks).
  static __device__ __forceinline__ int op_block(int m) {
    return m < Cfg::OP_BLK ? m : m - Cfg::OP_BLK;
  }

  __device__ __forceinline__ void init(const TileArgs& t, int wave_, int wave_m_, int lane) {
    wave = wave_;
    wave_m = wave_m_;
    const int64_t a_live = t.a_rows - t.a_row0;  // >= 1
    const int64_t w_live = t.w_rows - t.w_row0;  // >= 1
    if constexpr (!Cfg::A_CAST) ra = make_rsrc(t.A + t.a_row0 * t.K, a_live * t.K);
    rw = make_rsrc(t.W + t.w_row0 * t.K, w_live * t.K);
    if constexpr (!Cfg::OP_BF16 && !Cfg::A_CAST) {
      const int64_t G = t.K / Cfg::BK;
      rs = make_rsrc(t.SA + t.a_row0, (G * t.sa_ld - t.a_row0) * 4);
      s_stride = t.sa_ld * 4;
    }
    const int sub_r = lane >> 3;
    const int pc = lane & 7;
#pragma unroll
    for (int j = 0; j < Cfg::PER_WAVE; ++j) {
      const int m = op_block(j * Cfg::NWAVES + wave);
      const bool is_a = m < Cfg::A_BLK;
      const int r = (is_a ? m : m - Cfg::A_BLK) * 8 + sub_r;
      const int64_t live = is_a ? a_live : w_live;
      const int64_t rr = r < live ? r : live - 1;
      voff[j] = (uint32_t)(rr * t.K) + (uint32_t)(swz(r, pc) * 16);
    }
    // Lane i of the scale load fetches row (i & 3) * 16 + i / 4 of the wave's
    // rows (up to 64; rows past them are loaded and not used), so the scales
    // an MFMA column lane needs (rows c, 16 + c, 32 + c, 48 + c) sit side by
    // side in LDS.
    if constexpr (!Cfg::OP_BF16 && !Cfg::A_CAST) {
      const int64_t rs_row = wave_m_ * Cfg::WM + (lane & 3) * 16 + (lane >> 2);
      voff_s = (uint32_t)((rs_row < a_live ? rs_row : a_live - 1) * 4);
    }
    if constexpr (Cfg::W_ROWSCALE) {
      // Wave w loads the scales of weight rows 64*(w%4) .. +63 of the tile
      // (waves w and w+4 write the same values).
      const int64_t G = t.K / Cfg::BK;
      rsb = make_rsrc(t.SW + t.w_row0, (G * t.sw_ld - t.w_row0) * 4);
      sb_stride = t.sw_ld * 4;
      const int64_t sb_row = (wave_ % 4) * 64 + lane;
      voff_sb = (uint32_t)((sb_row < w_live ? sb_row : w_live - 1) * 4);
    }
    // L2 prefetch lines.  The XCD-aware tile order gives one XCD a block of
    // 4 tile rows x 8 tile columns, so 8 tiles share each 256-row A band and
    // 4 share each W band in that XCD's L2.  A tile therefore prefetches
    // only its share: A rows 32*(tn%8) .. +31 (wave 0, lanes 0..31) and W
    // rows 64*(tm%4) .. +63 (wave 1).  Every other lane repeats its wave's
    // first line, which the address unit merges into one request: a prefetch
    // costs 96 line requests per tile and chunk instead of 512.
    const int tm = (int)(t.a_row0 / Cfg::BM), tn = (int)(t.w_row0 / Cfg::BN);
    pf_a = wave != 1;
    int pr = pf_a ? 32 * (tn % 8) : 64 * (tm % 4);
    if (wave == 1 || (wave == 0 && lane < 32)) pr += lane;
    const int64_t plive = pf_a ? a_live : w_live;
    voff_pf = (uint32_t)((pr < plive ? pr : plive - 1) * t.K);
  }

  // L2 prefetch h (0 .. PF_LOADS-1) of this lane's line of chunk g: a 4-byte
  // direct-to-LDS load into the wave's landing slot, whose contents nobody
  // reads.  It is counted by vmcnt like the operand loads.
  __device__ __forceinline__ void prefetch(uint8_t* slot, int64_t g, int h) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(pf_a ? ra : rw, to_lds(slot), 4,
                                             voff_pf + (uint32_t)(h * 64), (int)(g * Cfg::BK), 0, 0);
  }

  // Load d (0 .. LOADS-1) of chunk g into `stage`.
  __device__ __forceinline__ void issue(uint8_t* stage, int64_t g, int d) const {
    if (d < Cfg::PER_WAVE) {
      const int m = op_block(d * Cfg::NWAVES + wave);
      const bool is_a = m < Cfg::A_BLK;
      const int dst = is_a ? m * 1024 : Cfg::A_BYTES + (m - Cfg::A_BLK) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? ra : rw, to_lds(stage + dst), 16, voff[d],
                                               (int)(g * Cfg::BK), 0, 0);
    } else if (!Cfg::OP_BF16 && !Cfg::A_CAST && d == Cfg::PER_WAVE) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, to_lds(stage + Cfg::A_BYTES + Cfg::B_BYTES + wave_m * 256), 4, voff_s,
          (int)(g * s_stride), 0, 0);
    } else if constexpr (Cfg::W_ROWSCALE) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsb,
          to_lds(stage + Cfg::A_BYTES + Cfg::B_BYTES + Cfg::SA_BYTES + (wave % 4) * 256), 4,
          voff_sb, (int)(g * sb_stride), 0, 0);
    }
  }
};

// The activation operand quantized on its way into LDS: the FP8 cast fused
// with the global-to-LDS transfer (why-be.co.kr as_center post 57820,
// hardware-suggestion passage: the cast done during the transfer instead of
// an HBM round trip of the codes).  Each K chunk of the tile's BF16 rows
// comes into registers, 8 lanes per row (16 values, 32 bytes each) and 64
// rows per round (few registers: the main loop holds 221 of the 256).  The
// 8 lanes of a row reduce its 1x128 group max-abs (DPP), apply the
// quantizer's rule (quant_rules.hpp: the same codes and scale as
// fp8q_quantize_act, bit for bit), and write the codes into the stage's A
// slot at the swizzled places the direct loads would fill, and the scale into
// the row-scale slot of the row's wave row.  Rows past the valid range are
// read from the last valid row, as in the loads (their results are never
// stored).  The code has no branch: lanes past the staged
// rows (a partial last round) redo the last staged row and write the same
// bytes to the same places, and the 8 lanes of a row all write its scale.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint16_t v2u16 __attribute__((ext_vector_type(2)));

// Max-abs of 16 BF16 values as BF16 magnitude bits (in the low half), by
// packed 16-bit integer max: for non-negative floats the integer order of the
// bit patterns is the numeric order, so this is exactly the max of |x|.
__device__ __forceinline__ uint32_t absmax16_bits(const uint4& p, const uint4& q) {
  const uint32_t m = 0x7FFF7FFFu;
  auto h = [](uint32_t w) { return __builtin_bit_cast(v2u16, w); };
  v2u16 r = __builtin_elementwise_max(h(p.x & m), h(p.y & m));
  r = __builtin_elementwise_max(r, __builtin_elementwise_max(h(p.z & m), h(p.w & m)));
  r = __builtin_elementwise_max(r, __builtin_elementwise_max(h(q.x & m), h(q.y & m)));
  r = __builtin_elementwise_max(r, __builtin_elementwise_max(h(q.z & m), h(q.w & m)));
  return r[0] > r[1] ? r[0] : r[1];
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
  return o > v ? o : v;
}

template <class Cfg>
struct ACaster {
  __amdgpu_buffer_rsrc_t rx;  // the tile's BF16 rows
  int a_last;                 // last valid row of the tile (only rows below ROWS matter)
  uint32_t row_bytes;         // 2K
  int row0;                   // this lane's row in round 0 (tid / 8)
  int oc;                     // which 16-value eighth of the row (= logical code column)
  uint4 raw[2];               // the loaded round's 16 BF16 values

  // LDS row of this lane in round r.
  __device__ __forceinline__ int row_of(int r) const {
    const int row = r * 64 + row0;
    return row < Cfg::ROWS ? row : Cfg::ROWS - 1;
  }

  __device__ __forceinline__ void init(const TileArgs& t, int tid) {
    const int64_t a_live = t.a_rows - t.a_row0;  // >= 1
    rx = make_rsrc(t.A + t.a_row0 * 2 * t.K, a_live * 2 * t.K);
    a_last = (int)(a_live < Cfg::ROWS ? a_live - 1 : Cfg::ROWS - 1);
    row_bytes = (uint32_t)(2 * t.K);
    row0 = tid >> 3;
    oc = tid & 7;
  }

  // BF16 values of chunk g, round r, into registers.
  __device__ __forceinline__ void load(int64_t g, int r) {
    const int row = row_of(r);
    const uint32_t rr = (uint32_t)(row < a_last ? row : a_last);
    const uint32_t voff = rr * row_bytes + (uint32_t)(oc * 32);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rx, voff + (uint32_t)(16 * p),
                                                         (int)(g * 256), 0);
      raw[p] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }

  // Codes and scale of the loaded round r into `stage`.
  __device__ __forceinline__ void cast_store(uint8_t* stage, int r) const {
    uint32_t ab = absmax16_bits(raw[0], raw[1]);
    ab = dpp_umax<kDppQuadXor1>(ab);       // the 8 lanes of a row: two quads,
    ab = dpp_umax<kDppQuadXor2>(ab);
    ab = dpp_umax<kDppRowHalfMirror>(ab);  // then each quad against the other
    const GroupRule rule = group_rule<Cfg::CAST_MODE>(__uint_as_float(ab << 16));
    const uint2 c0 = convert8<Cfg::CAST_MODE>(raw[0], rule);
    const uint2 c1 = convert8<Cfg::CAST_MODE>(raw[1], rule);
    const int row = row_of(r);
    // K bytes 16oc .. 16oc+15 of the row: logical 16-byte column oc.
    *reinterpret_cast<v4u*>(stage + row * 128 + swz(row, oc) * 16) = v4u{c0.x, c0.y, c1.x, c1.y};
    // Slot position of row rr of a wave row: (rr % 16) * 4 + rr / 16, the
    // order the scale loads of the other configurations produce.
    const int wm = row / Cfg::WM, rr = row % Cfg::WM;
    *reinterpret_cast<float*>(stage + Cfg::A_BYTES + Cfg::B_BYTES + wm * 256 +
                              ((rr & 15) * 4 + (rr >> 4)) * 4) = rule.s;
  }
};

// One 32-K half of a chunk for BF16 operands: fragment half h (the 16-byte
// piece q, or q + 4, of the 128-byte row, i.e. 8 BF16 values per lane) of the
// weight and activation fragments, accumulated into acc by the matrix core.
__device__ __forceinline__ v4f mfma_bf16_half(const v8i& w, const v8i& a, const v4f& acc,
                                              int h) {
  typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
  const v4i wh = h ? v4i{w[4], w[5], w[6], w[7]} : v4i{w[0], w[1], w[2], w[3]};
  const v4i ah = h ? v4i{a[4], a[5], a[6], a[7]} : v4i{a[0], a[1], a[2], a[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, wh),
                                                 __builtin_bit_cast(v8bf, ah), acc, 0, 0, 0);
}

// Promotion with row-scaled weights: acc += P * (s_a[row] * s_b[col]), the
// lane's 4 results having 4 weight rows.
__device__ __forceinline__ void promote_rows(v4f& acc, const v4f& p, float sa, const v4f& sb) {
  acc[0] = __builtin_fmaf(p[0], sa * sb[0], acc[0]);
  acc[1] = __builtin_fmaf(p[1], sa * sb[1], acc[1]);
  acc[2] = __builtin_fmaf(p[2], sa * sb[2], acc[2]);
  acc[3] = __builtin_fmaf(p[3], sa * sb[3], acc[3]);
}

// Promotion of one 16x16 chunk partial: acc += P * (s_a[row] * s_w).
__device__ __forceinline__ void promote(v4f& acc, const v4f& p, float mult) {
  acc[0] = __builtin_fmaf(p[0], mult, acc[0]);
  acc[1] = __builtin_fmaf(p[1], mult, acc[1]);
  acc[2] = __builtin_fmaf(p[2], mult, acc[2]);
  acc[3] = __builtin_fmaf(p[3], mult, acc[3]);
}

// Precise mode.  A fragment's 32 E4M3 codes widened to FP16, exactly (every
// E4M3 value, subnormals included, is an FP16 value; the conversion's scale
// operand 1.0 leaves it unscaled): FP16 word 2d + s holds byte 2s, 2s + 1 of
// code word d.  Quarter h (FP16 words 4h .. 4h+3) is fragment bytes 8h .. 8h+7,
// the 8 K values one lane gives one 16x16x32 MFMA; weight and activation
// quarters pair the same K.
typedef int v16i __attribute__((ext_vector_type(16)));
__device__ __forceinline__ v4i widen_quarter(const v8i& f, int h) {
  v4i o;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const int w = f[2 * h + d];
    o[2 * d] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    o[2 * d + 1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  }
  return o;
}

__device__ __forceinline__ v16i widen_frag(const v8i& f) {
  v16i o;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const v4i x = widen_quarter(f, h);
    o[4 * h] = x[0];
    o[4 * h + 1] = x[1];
    o[4 * h + 2] = x[2];
    o[4 * h + 3] = x[3];
  }
  return o;
}

__device__ __forceinline__ v4i quarter(const v16i& f, int h) {
  return v4i{f[4 * h], f[4 * h + 1], f[4 * h + 2], f[4 * h + 3]};
}

// One 32-K quarter of a chunk on widened codes: c + W_quarter . A_quarter.
__device__ __forceinline__ v4f mfma_wide16(const v4i& w, const v4i& a, const v4f& c) {
  typedef _Float16 v8h __attribute__((ext_vector_type(8)));
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, w),
                                                __builtin_bit_cast(v8h, a), c, 0, 0, 0);
}


// Block-scaled FP8 MFMA from zero: weight operand scaled by 2^(sw - 127),
// activation operand by 2^(byte i of sa - 127) (E8M0 bytes; op_sel picks the
// byte, so it must be an immediate: i is 0..3).
__device__ __forceinline__ v4f mfma_mx(const v8i& w, const v8i& a, int sw, int sa, int i) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  switch (i) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, z, 0, 0, 0, sw, 0, sa);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, z, 0, 0, 0, sw, 1, sa);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, z, 0, 0, 0, sw, 2, sa);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, z, 0, 0, 0, sw, 3, sa);
  }
}

// E8M0 byte of a power-of-two scale s >= 0 and the factor the matrix core
// cannot take: a normal s = 2^e is byte e + 127 (its FP32 exponent field) with
// factor 1; a subnormal s (e < -126) takes byte 0 (2^-127) and the exact
// factor s * 2^127; s = 0 (a flushed group, all codes zero) gives factor 0.
__device__ __forceinline__ int e8m0_byte(float s, float& factor) {
  const int b = (__float_as_int(s) >> 23) & 0xFF;
  factor = b == 0 ? s * 0x1p127f : 1.0f;
  return b;
}

// Computes one BM x BN output tile.  All lanes of the workgroup call it.
template <class Cfg>
__device__ __forceinline__ void gemm_tile(const TileArgs& t, uint8_t* smem) {
  constexpr int MB = Cfg::MB, NB = Cfg::NB, S = Cfg::STAGES;
  constexpr int RB = MB * Cfg::SUB;  // MFMA steps per weight row block
  constexpr bool WIDE = Cfg::WIDE16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_m = wave / Cfg::WAVES_N;
  const int wave_n = wave % Cfg::WAVES_N;
  const int r16 = lane & 15;   // fragment row within a 16-row block
  const int q = lane >> 4;     // which 16-byte piece pair of the 128-byte chunk
  const int64_t G = t.K / Cfg::BK;

  // Weight-scale row of this wave's weight rows (one 128-row block).
  const float* sw_row = nullptr;
  if constexpr (!Cfg::OP_BF16 && !Cfg::W_ROWSCALE) {
    int64_t wblk = (t.w_row0 + wave_n * Cfg::WN) / 128;
    const int64_t last_wblk = t.w_rows / 128 - 1;
    wblk = wblk < last_wblk ? wblk : last_wblk;
    sw_row = t.SW + wblk * G;
  }

  // Waves whose rows are all past the valid range skip the MFMA work.
  const bool wave_live =
      (wave_m * Cfg::WM < Cfg::ROWS) && (t.a_row0 + wave_m * Cfg::WM) < t.a_rows;

  // acc[i][j]: activation row block i (16 rows) x weight row block j.
  v4f acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Schedule of one chunk g (k = MFMA index, LAG = promotion lag):
  //   k = 0 ..         MFMAs of chunk g; the head loads of chunk g+S-1 go out
  //                    one every kDmaStep MFMAs from k = kDma0;
  //   k = kBar         wait for chunk g+1's loads, barrier: every wave has
  //                    finished reading stage g (its last weight fragment was
  //                    read at k = MB*(NB-1-BPF)) and chunk g+1 is in LDS;
  //   k > kBar         the tail loads of chunk g+S go into stage g, one per
  //                    MFMA, and once a fragment register has served its last
  //                    MFMA of chunk g it is refilled with chunk g+1's data,
  //                    so chunk g+1 starts with its operands in registers.
  // Step k is MFMA (weight row block j = k / MB, activation block i = k % MB):
  // one weight fragment serves MB consecutive MFMAs.  With BF16 operands a
  // block takes SUB = 2 MFMAs per chunk (the chunk's two 32-K halves): row
  // block j runs steps RB*j .. RB*j + RB - 1, first half h = 0 for the MB
  // activation blocks, then h = 1, so chained MFMAs are MB steps apart.
  // The matrix core therefore never waits for a chunk boundary: a wave that
  // arrives early at the barrier leaves the matrix core to its SIMD partner.
  // (Lag 1 with the activation cast: its registers come out of the partials'.)
  // In the precise mode (WIDE) a block's SUB = 4 MFMAs are consecutive steps
  // chained through their C operand (block b = k / SUB, i.e. activation block
  // i = b % MB of weight row block j = b / MB, quarter h = k % SUB); the
  // weight fragment of row block j is widened quarter by quarter in the steps
  // of its first block, and block b is promoted LAG steps after its last MFMA.
  constexpr int LAG = Cfg::OP_BF16 ? 0 : Cfg::A_CAST ? 1 : kPromoteLag;
  static_assert(!WIDE || LAG < Cfg::SUB, "two partial registers serve the precise mode");
  constexpr int KSTEPS = RB * NB + LAG;
  constexpr int kBar = RB * (NB - 1) - kBarLead;   // before the last row block
  constexpr int TAIL = KSTEPS - 1 - kBar;          // loads issued after the barrier
  constexpr int D1 = TAIL < Cfg::LOADS ? TAIL : Cfg::LOADS;
  // Weight fragments are read BPF row blocks ahead into a ring of BPF+1 slots.
  constexpr int BPF = kBPrefetch;
  constexpr int NBUF = BPF + 1;
  static_assert(kBar > RB * (NB - 1 - BPF), "the barrier follows the last weight read");
  static_assert(kBar < RB * (NB - 1), "the barrier precedes the last row block");
  // Step after which weight slot t (t < BPF) is free for chunk g+1's block t: the
  // last MFMA of the last block j < NB with j % NBUF == t, but not before the
  // barrier.
  auto next_b_step = [](int t) constexpr {
    int jt = t;
    while (jt + NBUF < NB) jt += NBUF;
    const int kt = RB * jt + RB - 1;
    return kt > kBar ? kt : kBar;
  };
  static_assert(kDma0 + (Cfg::LOADS - D1 - 1) * kDmaStep < kBar,
                "head loads are issued before the barrier");
  // The prefetches follow the head loads, kDmaStep MFMAs apart.
  constexpr int kPfAt = kDma0 + (Cfg::LOADS - D1) * kDmaStep;
  static_assert(kPfAt > kDma0 + (Cfg::LOADS - D1 - 1) * kDmaStep &&
                    kPfAt + (Cfg::PF_LOADS - 1) * kDmaStep < kBar,
                "prefetches go out after the head loads and before the barrier");

  // Activation cast: round r of chunk g+1 is quantized into chunk g+1's stage
  // at step cast_step(r) of chunk g, the last one a few steps before the
  // barrier that publishes chunk g+1.  Round 0's BF16 values are loaded right after
  // chunk g-1's barrier, ahead of the operand loads issued there, and round
  // r+1's right after round r's cast (one register set: a second one spills
  // the main loop), so each load has the steps up to its cast to arrive; the
  // casts are spread evenly over the chunk's cycle.  The stage of chunk g+1 is
  // free from chunk g's start on: its last reader, chunk g+1-S, ended before
  // chunk g-1's barrier.
  constexpr int CR = Cfg::CAST_ROUNDS;
  constexpr int kCastLast = kBar - 3;
  constexpr int kCastGap =
      CR > 1 ? (kCastLast / (CR - 1) < KSTEPS / CR ? kCastLast / (CR - 1) : KSTEPS / CR) : 0;
  auto cast_step = [](int r) constexpr { return kCastLast - (CR - 1 - r) * kCastGap; };
  static_assert(CR == 0 || (cast_step(0) >= 0 && kBar + 1 < KSTEPS),
                "the casts of a chunk precede its barrier");

  ChunkLoader<Cfg> ld;
  ld.init(t, wave, wave_m, lane);
  ACaster<Cfg> cs;
  if constexpr (Cfg::A_CAST) cs.init(t, threadIdx.x);
  // Chunk indices past the end are clamped to the last chunk: the extra loads
  // re-fetch L2-resident bytes into a stage nobody reads again, and keep the
  // number of loads in flight the same every iteration.
  const int64_t g_last = G - 1;
  uint8_t* const pf_slot = smem + S * Cfg::STAGE + wave * 256;
  constexpr int PFL = Cfg::PF_LOADS;
  // Loads issued after the last load of the chunk a barrier waits for: in
  // steady state S-2 whole chunks and S-1 iterations' prefetches.
  constexpr int kAfter = Cfg::LOADS * (S - 2) + PFL * (S - 1);
  // The prologue issues chunks 0 .. S-2 and the first D1 loads of chunk S-1
  // in the order S-1 steady-state iterations would (each chunk followed by
  // one iteration's prefetches), so every wait below counts the same loads.
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
#pragma unroll
    for (int d = 0; d < Cfg::LOADS; ++d)
      ld.issue(smem + s * Cfg::STAGE, s < g_last ? s : g_last, d);
    const int64_t gp = s - (S - 1) + kPfDist;
#pragma unroll
    for (int h = 0; h < PFL; ++h)
      ld.prefetch(pf_slot, gp < 0 ? 0 : (gp < g_last ? gp : g_last), h);
  }
#pragma unroll
  for (int d = 0; d < D1; ++d)
    ld.issue(smem + (S - 1) * Cfg::STAGE, S - 1 < g_last ? S - 1 : g_last, d);
  if constexpr (Cfg::A_CAST) {
#pragma unroll
    for (int r = 0; r < CR; ++r) {
      cs.load(0, r);
      cs.cast_store(smem, r);
    }
  }
  wait_vmcnt<kAfter + D1>();  // chunk 0 landed
  lds_barrier();
  if constexpr (Cfg::A_CAST) cs.load(g_last > 0 ? 1 : 0, 0);

  // activation fragments of the chunk (MFMA B operand); widened to FP16 in
  // the precise mode
  using AFrag = typename std::conditional<WIDE, v16i, v8i>::type;
  AFrag a[MB];
  v8i b[NBUF];   // weight fragments, a ring over row blocks (MFMA A operand)
  v16i bw;       // precise mode: the current row block's weight fragment, widened
  if (wave_live) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if constexpr (WIDE)
        a[i] = widen_frag(load_frag(smem, wave_m * Cfg::WM + i * 16 + r16, q));
      else
        a[i] = load_frag(smem, wave_m * Cfg::WM + i * 16 + r16, q);
    }
#pragma unroll
    for (int t = 0; t < BPF; ++t)
      b[t] = load_frag(smem + Cfg::A_BYTES, wave_n * Cfg::WN + t * 16 + r16, q);
  }

  int cur = 0;  // stage of chunk g
  for (int64_t g = 0; g < G; ++g) {
    const int nxt = cur + 1 == S ? 0 : cur + 1;    // stage of chunk g+1
    const int head = cur == 0 ? S - 1 : cur - 1;   // stage of chunk g+S-1
    const int64_t g_head = g + S - 1 < g_last ? g + S - 1 : g_last;
    const int64_t g_tail = g + S < g_last ? g + S : g_last;
    const int64_t g_pf = g + kPfDist < g_last ? g + kPfDist : g_last;
    const int64_t g_nxt = g + 1 < g_last ? g + 1 : g_last;
    const int64_t g_nxt2 = g + 2 < g_last ? g + 2 : g_last;
    uint8_t* const st_cur = smem + cur * Cfg::STAGE;
    uint8_t* const st_nxt = smem + nxt * Cfg::STAGE;
    uint8_t* const st_head = smem + head * Cfg::STAGE;
    if (!wave_live) {
#pragma unroll
      for (int d = D1; d < Cfg::LOADS; ++d) ld.issue(st_head, g_head, d);
#pragma unroll
      for (int h = 0; h < PFL; ++h) ld.prefetch(pf_slot, g_pf, h);
      if constexpr (Cfg::A_CAST) {
#pragma unroll
        for (int r = 0; r < CR; ++r) {
          cs.cast_store(st_nxt, r);
          if (r + 1 < CR) cs.load(g_nxt, r + 1);
        }
      }
      wait_vmcnt<kAfter>();
      lds_barrier();
      if constexpr (Cfg::A_CAST) cs.load(g_nxt2, 0);
#pragma unroll
      for (int d = 0; d < D1; ++d) ld.issue(st_cur, g_tail, d);
      cur = nxt;
      continue;
    }

    const uint8_t* Bs = st_cur + Cfg::A_BYTES;
    float mult[MB];
    int mx_w = 0, mx_a = 0;  // matrix-core scales: E8M0 bytes (weights; 4 activation blocks)
    v4f sa;
    // Row-scaled weights: the scales of row block j (this lane's 4 weight
    // rows) go into a 3-slot ring when the block's fragment is prefetched;
    // its last promotion comes before the slot is reused.
    const float* SBs =
        reinterpret_cast<const float*>(st_cur + Cfg::A_BYTES + Cfg::B_BYTES + Cfg::SA_BYTES);
    v4f sbv[3];
    if constexpr (!Cfg::OP_BF16) {
      const float* SAs =
          reinterpret_cast<const float*>(st_cur + Cfg::A_BYTES + Cfg::B_BYTES + wave_m * 256);
      sa = *reinterpret_cast<const v4f*>(SAs + 4 * r16);
      if constexpr (Cfg::W_ROWSCALE) {
        sbv[0] = *reinterpret_cast<const v4f*>(SBs + wave_n * Cfg::WN + 4 * q);
      } else if constexpr (Cfg::MX) {
        static_assert(MB <= 4, "one byte per activation block in a 32-bit scale register");
        float fw;
        mx_w = e8m0_byte(sw_row[g], fw);
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          float fa;
          mx_a |= e8m0_byte(sa[i], fa) << (8 * i);
          mult[i] = fa * fw;   // 1 unless a scale is below 2^-126
        }
      } else {
        const float sw = sw_row[g];
#pragma unroll
        for (int i = 0; i < MB; ++i) mult[i] = sa[i] * sw;
      }
    }
    // chunk partials: a ring over steps, or over blocks in the precise mode
    constexpr int PN = WIDE ? 2 : LAG + 1;
    v4f p[PN];
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      if (k < RB * NB) {
        const int i = WIDE ? (k / Cfg::SUB) % MB : k % MB;
        const int h = WIDE ? k % Cfg::SUB : (k / MB) % Cfg::SUB;
        const int j = k / RB;
        if (k % RB == 0 && j + BPF < NB)
          b[(j + BPF) % NBUF] = load_frag(Bs, wave_n * Cfg::WN + (j + BPF) * 16 + r16, q);
        if constexpr (Cfg::W_ROWSCALE) {
          static_assert(RB * (NB - 2) < kBar, "row scales are read before the barrier");
          if (k % RB == 0 && j + 1 < NB)
            sbv[(j + 1) % 3] =
                *reinterpret_cast<const v4f*>(SBs + wave_n * Cfg::WN + (j + 1) * 16 + 4 * q);
        }
        if constexpr (Cfg::OP_BF16) {
          acc[i][j] = mfma_bf16_half(b[j % NBUF], a[i], acc[i][j], h);
        } else if constexpr (WIDE) {
          if (i == 0) {
            const v4i x = widen_quarter(b[j % NBUF], h);
            bw[4 * h] = x[0];
            bw[4 * h + 1] = x[1];
            bw[4 * h + 2] = x[2];
            bw[4 * h + 3] = x[3];
          }
          const int pb = (k / Cfg::SUB) % 2;
          p[pb] = mfma_wide16(quarter(bw, h), quarter(a[i], h),
                              h == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : p[pb]);
        } else if constexpr (Cfg::MX) {
          p[k % (LAG + 1)] = mfma_mx(b[j % NBUF], a[i], mx_w, mx_a, i);
        } else {
          p[k % (LAG + 1)] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              b[j % NBUF], a[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int d = D1; d < Cfg::LOADS; ++d)
        if (k == kDma0 + (d - D1) * kDmaStep) ld.issue(st_head, g_head, d);
#pragma unroll
      for (int h = 0; h < PFL; ++h)
        if (k == kPfAt + h * kDmaStep) ld.prefetch(pf_slot, g_pf, h);
      if (k == kBar) {
        wait_vmcnt<kAfter>();  // chunk g+1 landed
        lds_barrier();
      }
      if (k < RB * NB) {
        // Chunk g+1's fragments go into registers as soon as their chunk-g
        // contents have served their last MFMA (and the barrier at kBar has
        // made chunk g+1 visible): a[i] after row block NB-1's last MFMA with
        // it, weight slot t after the last block of chunk g that uses it.
        const int i = WIDE ? (k / Cfg::SUB) % MB : k % MB;
        const int h = WIDE ? k % Cfg::SUB : (k / MB) % Cfg::SUB;
        const int j = k / RB;
        if (j == NB - 1 && h == Cfg::SUB - 1) {
          if constexpr (WIDE)
            a[i] = widen_frag(load_frag(st_nxt, wave_m * Cfg::WM + i * 16 + r16, q));
          else
            a[i] = load_frag(st_nxt, wave_m * Cfg::WM + i * 16 + r16, q);
        }
#pragma unroll
        for (int t = 0; t < BPF; ++t)
          if (k == next_b_step(t))
            b[t] = load_frag(st_nxt + Cfg::A_BYTES, wave_n * Cfg::WN + t * 16 + r16, q);
      }
      // (Issued before the tail loads, so that waiting for these BF16
      // values never waits for chunk g+S's operands.)
      if constexpr (Cfg::A_CAST)
        if (k == kBar + 1) cs.load(g_nxt2, 0);
#pragma unroll
      for (int d = 0; d < D1; ++d)
        if (k == kBar + 1 + d) ld.issue(st_cur, g_tail, d);
      // Keep the step order: MFMA k is issued before block k-LAG's
      // promotion.  Left free, the scheduler hoists the promotion above the
      // MFMA (to hand its result registers to MFMA k), which leaves it right
      // behind MFMA k-LAG+1 and stalls the wave on the matrix core's result.
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (WIDE) {
        // block bb's last MFMA was step kp
        const int kp = k - LAG;
        if (kp >= 0 && kp < RB * NB && kp % Cfg::SUB == Cfg::SUB - 1) {
          const int bb = kp / Cfg::SUB;
          if constexpr (Cfg::W_ROWSCALE)
            promote_rows(acc[bb % MB][bb / MB], p[bb % 2], sa[bb % MB], sbv[(bb / MB) % 3]);
          else
            promote(acc[bb % MB][bb / MB], p[bb % 2], mult[bb % MB]);
        }
      } else if constexpr (Cfg::W_ROWSCALE) {
        const int kp = k - LAG;
        if (kp >= 0)
          promote_rows(acc[kp % MB][kp / MB], p[kp % (LAG + 1)], sa[kp % MB], sbv[(kp / MB) % 3]);
      } else if constexpr (!Cfg::OP_BF16) {
        const int kp = k - LAG;
        if (kp >= 0) promote(acc[kp % MB][kp / MB], p[kp % (LAG + 1)], mult[kp % MB]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (Cfg::A_CAST) {
#pragma unroll
        for (int r = 0; r < CR; ++r)
          if (k == cast_step(r)) {
            cs.cast_store(st_nxt, r);
            if (r + 1 < CR) cs.load(g_nxt, r + 1);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    cur = nxt;
  }
  wait_vmcnt<0>();  // the trailing (clamped) loads have landed before the waves exit

  // Epilogue: in block (i, j) the lane holds activation row m = 16i + r16 and
  // weight rows n = 16j + 4q .. 16j + 4q + 3, i.e. 4 consecutive outputs.
  if (!wave_live) return;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int64_t m = t.a_row0 + wave_m * Cfg::WM + i * 16 + r16;
    if (m >= t.a_rows) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t n = t.w_row0 + wave_n * Cfg::WN + j * 16 + 4 * q;
      if (n >= t.w_rows) continue;
      if (t.out_bf16) {
        uint2 o;
        o.x = f32_to_bf16_bits(acc[i][j][0]) | (f32_to_bf16_bits(acc[i][j][1]) << 16);
        o.y = f32_to_bf16_bits(acc[i][j][2]) | (f32_to_bf16_bits(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(t.C) + m * t.ldc + n) = o;
      } else {
        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(t.C) + m * t.ldc + n) = acc[i][j];
      }
    }
  }
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::THREADS) void gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, const uint8_t* __restrict__ W,
    const float* __restrict__ SW, int64_t M, int64_t N, int64_t K, void* __restrict__ C,
    int out_bf16, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::LDS_BYTES];
  int tm, tn;
  xcd_tile(blockIdx.x, gridDim.x, tiles_n, tm, tn);
  TileArgs t;
  t.A = A;
  t.SA = SA;
  t.W = W;
  t.SW = SW;
  t.a_row0 = (int64_t)tm * Cfg::BM;
  t.a_rows = M;
  t.w_row0 = (int64_t)tn * Cfg::BN;
  t.w_rows = N;
  t.K = K;
  t.sa_ld = M;
  t.sw_ld = N;
  t.C = C;
  t.ldc = N;
  t.out_bf16 = out_bf16;
  gemm_tile<Cfg>(t, smem);
}

// Grouped variant, persistent: one workgroup per CU (the grid grows only if a
// workgroup would otherwise walk more than 64 tiles).  Each workgroup derives
// the whole schedule from the device offsets, in LDS, once: it ranks the
// experts by row count and orders them for a balanced, largest-first
// schedule (snake_position) when the tiles fill few rounds, takes a prefix
// sum of ceil(M_e / 256) in that order, and maps each of its own tiles to
// (expert, m-tile, n-tile), one tile per lane.  It then runs the tiles one
// after the other, each with the instantiation for its live row count.
// Paying the set-up once per CU rather than once per tile (a kernel of one
// workgroup per tile spent about 4 us per workgroup on launch and set-up
// that the single resident workgroup of a CU cannot overlap).

// Position of the expert of rank r (0 = most rows) among G experts dealt to
// the 8 XCD runs in snake order: ranks 0..7 go to runs 0..7, ranks 8..15 to
// runs 7..0, and so on; run b holds its experts in rank order, and the runs
// follow each other.  A bijection on [0, G).
__device__ __forceinline__ int snake_position(int r, int G) {
  const int round = r / kXcds, i = r % kXcds;
  const int bin = (round & 1) ? kXcds - 1 - i : i;
  const int full = G / kXcds, m = G % kXcds;
  const bool last_odd = (full & 1) != 0;  // direction of the partial last round
  int start = bin * full;
  for (int b = 0; b < bin; ++b) start += (m > 0 && (last_odd ? b >= kXcds - m : b < m)) ? 1 : 0;
  return start + round;
}

__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }

#ifdef FP8Q_DEBUG_CHECKS
// Set by a grouped launch that found invalid offsets (debug builds): read and
// cleared by the host entry points after their synchronization.
__device__ int g_offsets_error = 0;

hipError_t offsets_error_take(hipStream_t stream, int* flag) {
  const int zero = 0;
  hipError_t e = hipMemcpyFromSymbolAsync(flag, HIP_SYMBOL(g_offsets_error), sizeof(int), 0,
                                          hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e == hipSuccess && *flag)
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_offsets_error), &zero, sizeof(int), 0,
                          hipMemcpyHostToDevice);
  return e;
}
#endif
constexpr int kMaxExpertsLds = 1024;
constexpr int kGroupedThreads = 512;
constexpr int kGroupedLds =
    cmax(cmax(GroupedCfg<64, kS64>::LDS_BYTES, GroupedCfg<128, kS128>::LDS_BYTES),
         cmax(cmax(GroupedCfg<160, kS160>::LDS_BYTES, GroupedCfg<192, kS192>::LDS_BYTES),
              GroupedCfg<256, kS256>::LDS_BYTES));
static_assert(GroupedCfg<64, kS64>::THREADS == kGroupedThreads &&
                  GroupedCfg<256, kS256>::THREADS == kGroupedThreads,
              "all grouped configurations use the same workgroup");

// CAST: 0 = FP8 activation codes and scales in A / SA; 1 + scale mode = BF16
// activations in A (SA unused), quantized inside the tiles.  OP: kOpFp8, or
// kOpWide16 (the precise mode, with CAST = 0).
template <int CAST, int OP = kOpFp8>
__global__ __launch_bounds__(kGroupedThreads) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, int64_t M_total,
    const int32_t* __restrict__ off, int G, const uint8_t* __restrict__ W,
    const float* __restrict__ SW, int64_t N, int64_t K, void* __restrict__ C, int out_bf16,
    int tiles_n, int lpt_max_tiles) {
  constexpr int T = kGroupedThreads;
  constexpr int BM = 256;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kGroupedLds];
  static_assert((3 * kMaxExpertsLds + 1) * 4 <= kGroupedLds, "prefix scratch fits in LDS");
  static_assert(kMaxExpertsLds % 64 == 0, "one wave scans the experts");
  int* mt_prefix = reinterpret_cast<int*>(smem);  // [G + 1], reused by the tiles' rings
  int* rows_of = mt_prefix + kMaxExpertsLds + 1;  // [G] rows of expert e
  int* expert_at = rows_of + kMaxExpertsLds;      // [G] expert at tile-order position p
  auto mtiles = [](int rows) { return rows > 0 ? (rows + BM - 1) / BM : 0; };

  // Number of real tiles, computed by every wave on its own from the offsets
  // (a lane sum and a wave reduction, no barrier), so that workgroups without
  // a tile leave before any LDS work.
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The same pass validates the offsets (0 = off[0] <= ... <= off[G] <=
  // M_total): every wave of every workgroup reads the same values and comes
  // to the same verdict, and with invalid offsets the whole launch returns
  // here, before any load or store.
  int sum_mt = 0;
  bool bad = lane == 0 && (off[0] != 0 || (int64_t)off[G] > M_total);
  for (int e = lane; e < G; e += 64) {
    const int lo = off[e], hi = off[e + 1];
    bad = bad || hi < lo;
    sum_mt += mtiles(hi - lo);
  }
  if (__ballot(bad) != 0) {
#ifdef FP8Q_DEBUG_CHECKS
    if (blockIdx.x == 0 && tid == 0) g_offsets_error = 1;
#endif
    return;
  }
  for (int d = 32; d >= 1; d >>= 1) sum_mt += __shfl_xor(sum_mt, d);
  // (equal in every lane; readfirstlane keeps everything derived from it scalar)
  const int total = __builtin_amdgcn_readfirstlane(sum_mt) * tiles_n;  // real tiles
  // Persistent schedule.  XCD x (= workgroup id mod 8) takes a contiguous run
  // of the real tiles, [x*q8 + min(x, r8), ...), so the n-tiles of one expert
  // share that expert's rows of A in one L2.  The K8 workgroups of an XCD walk
  // its run in rounds of K8 tiles in snake order (workgroup k takes run
  // position k in even rounds and K8-1-k in odd ones), which pairs the
  // largest tiles of a largest-first order with the smallest.  The host sizes
  // the grid so that no workgroup has more than 64 rounds.
  const int bid = blockIdx.x;
  const int K8 = gridDim.x / kXcds;
  const int x = bid % kXcds, k = bid / kXcds;
  const int q8 = total / kXcds, r8 = total % kXcds;
  const int run0 = x * q8 + (x < r8 ? x : r8);
  const int len = q8 + (x < r8 ? 1 : 0);
  if (k >= len) return;  // no tile for this workgroup

  for (int e = tid; e < G; e += T) rows_of[e] = off[e + 1] - off[e];
  __syncthreads();
  // Tile order.  When the tiles fill only a few rounds of the chip
  // (lpt_max_tiles = 4 per CU), the tail of the last round decides the time:
  // experts ranked by row count (largest first, ties by index) are dealt to
  // the 8 XCD runs in snake order, and each run lists its experts largest
  // first, so every XCD gets a similar share of the rows and its CUs take the
  // largest tiles first.  With many rounds, the expert order is kept: it mixes
  // tiles of different row counts (different MFMA-to-HBM ratios) in time.
  // Either way, each expert's tiles stay in one XCD run and share its L2
  // (exactly so when the runs hold equal tile counts, as with one m-tile per
  // expert).
  const bool lpt = total <= lpt_max_tiles;
  for (int e = tid; e < G; e += T) {
    int p = e;
    if (lpt) {
      const int ce = rows_of[e];
      int r = 0;
      for (int j = 0; j < G; ++j) {
        const int cj = rows_of[j];
        r += (cj > ce || (cj == ce && j < e)) ? 1 : 0;
      }
      p = snake_position(r, G);
    }
    expert_at[p] = e;
  }
  __syncthreads();

  // Prefix over tile-order positions of the number of BM-row tiles, by one
  // wave: lane l covers positions 16l .. 16l+15 (a lane sum, a shuffle scan
  // over the lanes, then the lane's 16 prefix values).
  if (tid < 64) {
    constexpr int PL = kMaxExpertsLds / 64;
    const int p0 = lane * PL;
    int sum = 0;
    for (int i = 0; i < PL; ++i)
      if (p0 + i < G) sum += mtiles(rows_of[expert_at[p0 + i]]);
    int inc = sum;
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(inc, d);
      if (lane >= d) inc += v;
    }
    int run = inc - sum;
    if (lane == 0) mt_prefix[0] = 0;
    for (int i = 0; i < PL; ++i)
      if (p0 + i < G) {
        run += mtiles(rows_of[expert_at[p0 + i]]);
        mt_prefix[p0 + i + 1] = run;
      }
  }
  __syncthreads();
  // Lane r of every wave maps this workgroup's round-r tile to (expert,
  // m-tile, n-tile): tile-order position p with prefix[p] <= m-tile index <
  // prefix[p+1].  Real tiles are numbered in tile order, m-tile, then n-tile
  // fastest.
  int my_e = 0, my_mt = 0, my_tn = 0;
  const int j = lane * K8 + ((lane & 1) ? K8 - 1 - k : k);
  const bool has = j < len;
  if (has) {
    const int id = run0 + j;
    const int mt_global = id / tiles_n;
    my_tn = id % tiles_n;
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (mt_prefix[mid] <= mt_global) lo = mid; else hi = mid;
    }
    my_e = expert_at[lo];
    my_mt = mt_global - mt_prefix[lo];
  }
  // Rounds with a tile are a prefix of the lanes (j grows with the lane).
  const int n_mine = __builtin_popcountll(__ballot(has));
  __syncthreads();  // the prefix scratch is overwritten by the tiles' rings

  for (int r = 0; r < n_mine; ++r) {
    const int e = __builtin_amdgcn_readlane(my_e, r);
    const int mt = __builtin_amdgcn_readlane(my_mt, r);
    const int tn = __builtin_amdgcn_readlane(my_tn, r);
    const int64_t r0 = off[e];
    const int64_t r1 = off[e + 1];
    TileArgs t;
    t.A = A;
    t.SA = SA;
    t.W = W + (int64_t)e * N * K;
    t.SW = SW + (int64_t)e * (N / 128) * (K / 128);
    t.a_row0 = r0 + (int64_t)mt * BM;
    t.a_rows = r1;
    t.w_row0 = (int64_t)tn * kGroupedBN;
    t.w_rows = N;
    t.K = K;
    t.sa_ld = M_total;
    t.sw_ld = N;
    t.C = C;
    t.ldc = N;
    t.out_bf16 = out_bf16;
    const int64_t live = r1 - t.a_row0;  // 1 .. (>= 256 when more m-tiles follow)
    if (live <= 64)
      gemm_tile<GroupedCfg<64, kS64, CAST, OP>>(t, smem);
    else if (live <= 128)
      gemm_tile<GroupedCfg<128, kS128, CAST, OP>>(t, smem);
    else if (live <= 160)
      gemm_tile<GroupedCfg<160, kS160, CAST, OP>>(t, smem);
    else if (live <= 192)
      gemm_tile<GroupedCfg<192, kS192, CAST, OP>>(t, smem);
    else
      gemm_tile<GroupedCfg<256, kS256, CAST, OP>>(t, smem);
    __syncthreads();  // the next tile's loads reuse the ring
  }
}

hipError_t launch_gemm_bf16(const void* a, const void* w, int64_t M, int64_t N, int64_t K,
                            void* c, int out_bf16, hipStream_t stream) {
  using Cfg = DenseBf16Cfg;
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles_m = (M + Cfg::BM - 1) / Cfg::BM;
  const int64_t tiles_n = (N + Cfg::BN - 1) / Cfg::BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  // Operand rows are 2K bytes: the kernel's K is the row length in bytes.
  hipLaunchKernelGGL(gemm_kernel<Cfg>, dim3((unsigned)tiles), dim3(Cfg::THREADS), 0, stream,
                     static_cast<const uint8_t*>(a), nullptr, static_cast<const uint8_t*>(w),
                     nullptr, M, N, 2 * K, c, out_bf16, (int)tiles_n);
  return hipGetLastError();
}

template <class Cfg>
static hipError_t launch_rowscaled_cfg(const uint8_t* a_q, const float* a_s, const uint8_t* b_q,
                                       const float* b_s, int64_t M, int64_t N, int64_t K, void* c,
                                       int out_bf16, hipStream_t stream) {
  const int64_t tiles_m = (M + Cfg::BM - 1) / Cfg::BM;
  const int64_t tiles_n = (N + Cfg::BN - 1) / Cfg::BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_kernel<Cfg>, dim3((unsigned)tiles), dim3(Cfg::THREADS), 0, stream, a_q,
                     a_s, b_q, b_s, M, N, K, c, out_bf16, (int)tiles_n);
  return hipGetLastError();
}

hipError_t launch_gemm_rowscaled(const uint8_t* a_q, const float* a_s, const uint8_t* b_q,
                                 const float* b_s, int64_t M, int64_t N, int64_t K, void* c,
                                 int out_bf16, int precise, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (precise)
    return launch_rowscaled_cfg<RowScaledWideCfg>(a_q, a_s, b_q, b_s, M, N, K, c, out_bf16,
                                                  stream);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipGetLastError();
  // Rounds of tiles over the CUs times the tile width: the 224-row weight
  // tiles when they finish sooner by that measure.
  const int64_t tm = (M + 255) / 256;
  const int64_t r256 = (tm * ((N + 255) / 256) + cus - 1) / cus;
  const int64_t r224 = (tm * ((N + 223) / 224) + cus - 1) / cus;
  if (r224 * 224 < r256 * 256)
    return launch_rowscaled_cfg<RowScaled224Cfg>(a_q, a_s, b_q, b_s, M, N, K, c, out_bf16, stream);
  return launch_rowscaled_cfg<RowScaledCfg>(a_q, a_s, b_q, b_s, M, N, K, c, out_bf16, stream);
}

hipError_t launch_gemm(const uint8_t* a_q, const float* a_s, const uint8_t* w_q,
                       const float* w_s, int64_t M, int64_t N, int64_t K, void* c, int out_bf16,
                       int mode, hipStream_t stream) {
  using Cfg = DenseCfg;
  static_assert(DenseWideCfg::BM == Cfg::BM && DenseWideCfg::BN == Cfg::BN, "same tiles");
  static_assert(DenseMxCfg::BM == Cfg::BM && DenseMxCfg::BN == Cfg::BN, "same tiles");
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles_m = (M + Cfg::BM - 1) / Cfg::BM;
  const int64_t tiles_n = (N + Cfg::BN - 1) / Cfg::BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  // mode 0: FP8 MFMA; 1: the precise mode; 2: scales applied by the matrix core
  auto kern = mode == 1 ? gemm_kernel<DenseWideCfg>
              : mode == 2 ? gemm_kernel<DenseMxCfg> : gemm_kernel<Cfg>;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(Cfg::THREADS), 0, stream, a_q, a_s, w_q,
                     w_s, M, N, K, c, out_bf16, (int)tiles_n);
  return hipGetLastError();
}

// BF16 activations x quantized inside the dense GEMM (scale mode `mode`).
hipError_t launch_gemm_cast(const void* x, const uint8_t* w_q, const float* w_s, int64_t M,
                            int64_t N, int64_t K, void* c, int out_bf16, int mode,
                            hipStream_t stream) {
  using Cfg = DenseCastCfg<0>;
  static_assert(DenseCastCfg<1>::BM == Cfg::BM && DenseCastCfg<1>::BN == Cfg::BN, "same tiles");
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles_m = (M + Cfg::BM - 1) / Cfg::BM;
  const int64_t tiles_n = (N + Cfg::BN - 1) / Cfg::BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  auto kern = mode == 0 ? gemm_kernel<DenseCastCfg<0>> : gemm_kernel<DenseCastCfg<1>>;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(Cfg::THREADS), 0, stream,
                     static_cast<const uint8_t*>(x), nullptr, w_q, w_s, M, N, K, c, out_bf16,
                     (int)tiles_n);
  return hipGetLastError();
}

// cast = 0: a holds FP8 codes with scales a_s; cast = 1 + mode: a holds BF16
// activations quantized inside the kernel (a_s unused); cast = -1: FP8 codes
// through the precise mode.
static hipError_t launch_grouped(const uint8_t* a, const float* a_s, int64_t M_total,
                                 const int32_t* off, int G, const uint8_t* w_q,
                                 const float* w_s, int64_t N, int64_t K, void* c, int out_bf16,
                                 int cast, hipStream_t stream) {
  if (M_total == 0 || N == 0) return hipSuccess;
  if (G > kMaxExpertsLds) return hipErrorInvalidValue;
  const int64_t tiles_n = (N + kGroupedBN - 1) / kGroupedBN;
  // sum_e ceil(M_e / 256) <= floor(M_total / 256) + G
  const int64_t max_mtiles = M_total / 256 + G;
  const int64_t tiles = max_mtiles * tiles_n;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipGetLastError();
  // Persistent grid: one workgroup per CU (LDS allows one), 8 per XCD
  // round, and enough of them that no workgroup walks more than 64 rounds of
  // its XCD's run (at most ceil(tiles / 8) tiles).
  const int64_t per_xcd = (tiles + kXcds - 1) / kXcds;
  int64_t k8 = (cus + kXcds - 1) / kXcds;
  if (k8 < (per_xcd + 63) / 64) k8 = (per_xcd + 63) / 64;
  const int64_t grid = k8 * kXcds;
  // The largest-first order applies up to 4 tiles per CU of the device.
  auto kern = cast == -1  ? grouped_gemm_kernel<0, kOpWide16>
              : cast == 0 ? grouped_gemm_kernel<0>
              : cast == 1 ? grouped_gemm_kernel<1>
                          : grouped_gemm_kernel<2>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kGroupedThreads), 0, stream, a, a_s,
                     M_total, off, G, w_q, w_s, N, K, c, out_bf16, (int)tiles_n, 4 * cus);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const uint8_t* a_q, const float* a_s, int64_t M_total,
                               const int32_t* off, int G, const uint8_t* w_q, const float* w_s,
                               int64_t N, int64_t K, void* c, int out_bf16, int precise,
                               hipStream_t stream) {
  return launch_grouped(a_q, a_s, M_total, off, G, w_q, w_s, N, K, c, out_bf16,
                        precise ? -1 : 0, stream);
}

hipError_t launch_grouped_gemm_cast(const void* x, int64_t M_total, const int32_t* off, int G,
                                    const uint8_t* w_q, const float* w_s, int64_t N, int64_t K,
                                    void* c, int out_bf16, int mode, hipStream_t stream) {
  return launch_grouped(static_cast<const uint8_t*>(x), nullptr, M_total, off, G, w_q, w_s, N,
                        K, c, out_bf16, 1 + mode, stream);
}

}  // namespace fp8q
