// Perturbed LSTM gate product + fused cell update for bf16 models on gfx950 matrix cores.
//
// One launch per (layer, timestep) computes, for every probe pair of a chunk, the gate
// pre-activations of both perturbed models (theta + eps p_i and theta - eps p_i),
//   G = (W_ih +- eps P_ih) x_t + (W_hh +- eps P_hh) h_{t-1} + (b +- eps p_b),
// and applies the LSTM cell to them in registers. This is the complete recurrent forward pass at
// perturbed weights that the method evaluates (alex-wiki source note on arXiv 2505.17852,
// "Method"), with Rademacher perturbations (pith.science review, "What carries the argument").
//
// The perturbed weight tile is never stored to memory. Each thread loads 8 stored weights w of
// one row, forms both candidates bf16(w + eps) and bf16(w - eps) in registers (one float add each
// and the packed round-to-nearest-even conversion), and the probe's sign bit picks one candidate
// per model: the +eps model takes the one the sign selects, the -eps model the other. The result
// goes to LDS. Sign bits come from per-chunk tables of Philox words (one 32-bit word per row and
// 32-column chunk, chunk-major), so both models of a pair share one weight load and one sign
// word.
//
// Workgroup tile (512 threads = 8 waves of 64 lanes, two per SIMD):
//   rows    128 gate rows = 32 hidden units x 4 gates, interleaved (local row 4u + g is gate g of
//           unit u) so that each lane's 16x16 accumulator holds all four gates of one unit;
//   columns 256 batch columns of the +eps model and the same 256 of the -eps model;
//   waves   (model, column quarter): each wave owns 128 x 64 = 8 x 4 MFMA 16x16x32 tiles
//           (128 accumulator registers per lane).
// K loop over the concatenated reduction [x_t ; h_{t-1}] in chunks of 32, software-pipelined:
//   * activations (stored k-chunk-major, so a 16-column fragment is 1 KB of contiguous memory)
//     go straight from global memory into the MFMA operand registers of the wave that uses them
//     (each column belongs to one wave), in a 4-deep register ring, three chunks ahead;
//   * the stored weights (read from a tile-major copy, in which a tile's 128 rows of one chunk
//     are 8 KB of contiguous memory) and sign words of chunks c+5 and c+6 are requested together
//     in odd steps into a register ring, and chunk c+4 is selected into LDS in step c, after row
//     group 5;
//   * the selected tiles of both models live in an 8-stage LDS ring; fragments are read two row
//     groups ahead of the MFMAs that use them; a barrier follows the select in every fourth step.
// The cell state stays in accumulator order (tile-private, 16 bytes per lane and row group), and
// h leaves as whole 64-byte column segments, regrouped in registers by lane exchanges.
// The 1-D grid is ordered so that the 32 workgroups resident on one XCD at a time cover 16 row
// tiles x 2 column blocks (or 8 x 4; the last row group of a column group may be shorter), which
// keeps their shared weight and activation chunks in that XCD's L2.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels_common.h"

namespace cdrge {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kGateThreads = 512;
constexpr int kUnitsPerTile = 32;
constexpr int kTileRows = 4 * kUnitsPerTile;   // 128 gate rows
constexpr int kTileCols = 256;                 // batch columns per model
constexpr int kKChunk = 32;
constexpr int kAStageBytes = 2 * kTileRows * 64;   // both models' 128 x 32 bf16 tiles
constexpr int kAStages = 8;
constexpr int kBRing = 4;                          // activation register ring (chunks)
// K-step phases (see the step of k_lstm_gates_bf16): every request, or the last two groups of four
constexpr int kAll = 0, kPenult = 1, kLast = 2;
constexpr int kPhasedMaxChunks = 64;  // longest reduction (in chunks) run on the phased instance
// Workgroups resident on one XCD at a time (one per CU, 32 per XCD) cover group_rows row tiles x
// group_cols column blocks (16 x 2 or 8 x 4, chosen by the host), so that each activation chunk
// is fetched into that XCD's L2 once for group_rows workgroups and each weight chunk once for
// group_cols.
constexpr size_t kGateBiasOffset = size_t(kAStages) * kAStageBytes;
constexpr size_t kGateLdsBytes = kGateBiasOffset + sizeof(float) * 2 * 4 * kUnitsPerTile;  // + gate biases

// Byte offset of 16-byte piece p (k = 8p..8p+7) of row r in a tile of 64-byte rows. Pieces are
// XOR-swizzled with f(r) = (r >> 1) & 3, which depends on r mod 8 only (a fragment of 16 rows
// starts 1 KB further). Measured with the LDS counters on gfx950: the A-operand read (lane l:
// row l % 16, piece l / 16) then takes 4 LDS cycles per instruction with no bank conflict, where
// f(r) = ((r >> 1) ^ ((r >> 3) & 1)) & 3, r & 3, (r >> 2) & 3 or no swizzle take 8 (4 of them
// conflict cycles); the select write (thread t: row t / 4, piece t % 4) is conflict-free with
// every one of them.
__device__ __forceinline__ int piece_offset(int r, int p) {
  return r * 64 + 16 * (p ^ ((r >> 1) & 3));
}

struct GateArgs {
  const uint16_t* w_ih;    // W_ih [4H][in], bf16 parameters, in the tile-major copy of k_tile_gate_weights
  const uint16_t* w_hh;    // W_hh [4H][H], likewise
  const uint32_t* sg_ih;   // sign words of W_ih for the chunk's pairs, [pairs][in / 32][4H]
  const uint32_t* sg_hh;   // sign words of W_hh, [pairs][H / 32][4H]
  const uint16_t* x_in;    // input of this layer at t, [in / 32][ncols_pad][32] (k-chunk-major)
  const uint16_t* h_prev;  // this layer's h_{t-1}, [H / 32][ncols_pad][32] (unused when first)
  uint16_t* h_out;         // this layer's h_t, [H / 32][ncols_pad][32]
  float* c_tile;           // this layer's cell state in accumulator order, 64 KB per tile
  const float* bias_m;     // per-model perturbed gate bias [2P][L][4H]
  float eps;
  int in, H, B, L, layer, first, ncols_pad;
  int n_row_tiles, n_col_blocks, n_pairs, swizzle, group_rows, group_cols;
};

// Row tile / column block / pair of this workgroup (see the header comment for the XCD order).
__device__ __forceinline__ void gate_tile_of_block(const GateArgs& a, int& rt, int& cb, int& pr) {
  const int L = blockIdx.x;
  int rtile, cw;
  if (a.swizzle) {
    // Workgroups are dealt to the 8 XCDs round-robin; v enumerates one XCD's workgroups in
    // dispatch order (a bijection when the grid is a multiple of 8, which the host guarantees).
    // v runs through the column blocks group_cols at a time; within such a column group, each
    // run of group_rows * group_cols workgroups covers group_rows row tiles x group_cols column
    // blocks, and when the row tiles do not divide by group_rows the rest form one shorter group.
    // A group may start on one XCD and end on the next.
    const int n = gridDim.x;
    const int v = (L & 7) * (n >> 3) + (L >> 3);
    const int gr = a.group_rows, gc = a.group_cols, gsz = gr * gc;
    const int per_cg = a.n_row_tiles * gc;
    const int cg = v / per_cg, r = v - cg * per_cg;
    const int n_full = a.n_row_tiles / gr;
    if (r < n_full * gsz) {
      const int g = r / gsz, q = r - g * gsz;
      rtile = g * gr + q % gr;
      cw = cg * gc + q / gr;
    } else {
      const int rem = a.n_row_tiles - n_full * gr, q = r - n_full * gsz;  // rem > 0 here
      rtile = n_full * gr + q % rem;
      cw = cg * gc + q / rem;
    }
  } else {
    rtile = L % a.n_row_tiles;
    cw = L / a.n_row_tiles;
  }
  rt = rtile;
  cb = cw % a.n_col_blocks;
  pr = cw / a.n_col_blocks;
}

// Tile-major copy of one gate weight matrix W [4H][cols] (bf16, cols a multiple of 32) for
// k_lstm_gates_bf16. Block (rt, cc) holds row tile rt (its local row 4u + g is gate g of unit
// 32 rt + u, i.e. row g H + 32 rt + u of W) and columns 32 cc .. 32 cc + 31, row-major: 128 x 32
// values, 8 KB of contiguous memory; blocks are ordered rt-major. One thread per 16 bytes.
__global__ void k_tile_gate_weights(const uint16_t* __restrict__ w, int H, int cols, uint16_t* __restrict__ wt) {
  const int nch = cols / kKChunk;
  const int64_t pieces = int64_t(4) * H * cols / 8;
  for (int64_t o = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; o < pieces;
       o += int64_t(gridDim.x) * blockDim.x) {
    const int64_t blk = o >> 9;  // 512 pieces per block
    const int pc = static_cast<int>(o & 511);
    const int rt = static_cast<int>(blk / nch), cc = static_cast<int>(blk - int64_t(rt) * nch);
    const int ra = pc >> 2, q = pc & 3;
    const int64_t row = int64_t(ra & 3) * H + int64_t(kUnitsPerTile) * rt + (ra >> 2);
    *reinterpret_cast<uint4*>(wt + 8 * o) =
        *reinterpret_cast<const uint4*>(w + row * cols + int64_t(kKChunk) * cc + 8 * q);
  }
}

// kExact (exact-perturbation bf16): stage half 0 holds the stored weights W and half 1 the bf16
// operand eps' P (eps' = a.eps, a bf16 value; P = +-1 from the sign words); every wave multiplies
// both into its accumulators, the -eps model with the sign bits of eps' P flipped in registers,
// so that G = W [x; h] +- eps' P [x; h] with no rounding of the perturbed weight. Twice the
// matrix-core work; A fragments are read one row group ahead (two rings of two) to stay within
// the register budget of two waves per SIMD.
//
// kPhased: the chunk count (in + H, or in alone at the first timestep, over 32) is a multiple of
// 4 and at least 8, and the last two groups of four K steps leave out the requests past the end
// (the host picks the instance, for short reductions; one code path per instance keeps the
// register budget).
template <bool kExact, bool kPhased>
__global__ __launch_bounds__(kGateThreads, 1) void k_lstm_gates_bf16(GateArgs a) {
  extern __shared__ __align__(16) uint16_t smem[];
  char* As = reinterpret_cast<char*>(smem);  // [8 stages][model][128 rows][64 B], swizzled

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
  const int side = wave >> 2, cq = wave & 3;
  const int H = a.H;
  int rt, cb, pr;
  gate_tile_of_block(a, rt, cb, pr);
  const int u0 = rt * kUnitsPerTile;
  const int bcol0 = cb * kTileCols;
  const int m_out = 2 * pr + side;

  // ---- weight select: thread owns local row ra = tid/4 (4 lanes per row), piece q = tid%4 ----
  const int q = tid & 3;
  const int ra = tid >> 2;
  const int grow = (ra & 3) * H + u0 + (ra >> 2);
  // Weights come from the tile-major copies (k_tile_gate_weights): the 128 rows x 32 columns of
  // this row tile and one chunk are 8 KB of contiguous memory, and this thread's 16 bytes (row ra,
  // columns 8q..8q+7) are at element 8 tid of the block, so each wave reads 1 KB of contiguous
  // weights per chunk (eight whole cache lines rather than sixteen halves).
  // (a wave-uniform base per chunk plus a 32-bit per-lane byte offset)
  const char* wt_x = reinterpret_cast<const char*>(a.w_ih + static_cast<int64_t>(rt) * (a.in / kKChunk) * kTileRows * kKChunk);
  const char* wt_h = reinterpret_cast<const char*>(a.w_hh + static_cast<int64_t>(rt) * (H / kKChunk) * kTileRows * kKChunk);
  const uint32_t wt_lane = 16u * static_cast<uint32_t>(tid);
  // sign words of row grow for this pair: one 32-bit word per 32-column chunk, chunk-major, so
  // the 128 rows of a tile read 4 runs of 32 consecutive words per chunk
  const uint32_t* sgx = a.sg_ih + static_cast<int64_t>(pr) * (a.in / kKChunk) * (4 * H) + grow;
  const uint32_t* sgh = a.sg_hh + static_cast<int64_t>(pr) * (H / kKChunk) * (4 * H) + grow;

  // ---- activation operand of this wave: lane holds column 64 cq + 16 j + lane % 16 of model
  // m_out, k piece lane / 16 (the MFMA B layout). Activations are stored k-chunk-major, element
  // (column, k) at ((k / 32) ncols_pad + column) 32 + k % 32, so the 16 columns of one fragment
  // are 1 KB of contiguous memory. Columns past the batch read the padding or the next model's
  // columns (results unused). Element offsets are 32-bit: the host guarantees that the padded
  // column count times max(in, H) fits.
  const int kp = lane >> 4;
  const uint32_t gcol0 = static_cast<uint32_t>(m_out * a.B + bcol0 + 64 * cq + (lane & 15));
  const uint32_t boff = gcol0 * kKChunk + 8 * kp;
  const int64_t chunk_stride = static_cast<int64_t>(a.ncols_pad) * kKChunk;

  const int kx = a.in / kKChunk;
  const int kh = a.first ? 0 : H / kKChunk;
  const int nch = kx + kh;

  auto load_w = [&](int c, uint4& w_out, uint32_t& word_out) {
    const bool xpart = c < kx;
    const int cc = xpart ? c : c - kx;
    const char* w = (xpart ? wt_x : wt_h) + static_cast<int64_t>(cc) * (kTileRows * kKChunk * 2);
    w_out = *reinterpret_cast<const uint4*>(w + wt_lane);
    word_out = (xpart ? sgx : sgh)[static_cast<int64_t>(cc) * (4 * H)];
  };
  // Selects the probe's weights for row ra of one chunk (8 bf16 weights wv and the row's sign
  // word of that chunk) and writes both models' tiles to LDS stage `stage`. The two candidates
  // bf16(w + eps) and bf16(w - eps) are formed here (one float add each, then the packed
  // round-to-nearest-even conversion) and the sign bit picks one per model.
  const float eps = a.eps;
  const uint32_t eps2 = (__float_as_uint(eps) >> 16) * 0x00010001u;  // bf16 eps' in both halves
  auto form_w = [&](const uint4& wv, uint32_t word, int stage) {
    // Piece q covers columns 8q..8q+7 of the 32-column word: pairs 4q..4q+3, which read bits
    // 4q+p (even column) and 16+4q+p (odd column).
    const uint32_t t4 = word >> (4 * q);
    const uint32_t w2[4] = {wv.x, wv.y, wv.z, wv.w};
    uint32_t plus[4], minus[4];
    if constexpr (kExact) {
      // half 0: W as stored; half 1: eps' P (sign bit set where the probe sign is -1)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        plus[p] = w2[p];
        minus[p] = eps2 | ((t4 << (15 - p)) & 0x80008000u);
      }
      char* st = As + stage * kAStageBytes;
      *reinterpret_cast<uint4*>(st + piece_offset(ra, q)) = make_uint4(plus[0], plus[1], plus[2], plus[3]);
      *reinterpret_cast<uint4*>(st + piece_offset(kTileRows + ra, q)) = make_uint4(minus[0], minus[1], minus[2], minus[3]);
      return;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float lo = __uint_as_float(w2[p] << 16), hi = __uint_as_float(w2[p] & 0xffff0000u);
      const f32x2 vp = {lo + eps, hi + eps}, vm = {lo - eps, hi - eps};
      const uint32_t pv = __builtin_bit_cast(uint32_t, __builtin_convertvector(vp, bf16x2));
      const uint32_t mv = __builtin_bit_cast(uint32_t, __builtin_convertvector(vm, bf16x2));
      // bits p and p+16 moved to 15 and 31, then replicated over each half-word
      const uint32_t mk = __builtin_amdgcn_perm(0u, t4 << (15 - p), 0x09090808u);
      plus[p] = (mk & mv) | (~mk & pv);   // sign -1: +eps model takes w - eps
      minus[p] = (mk & pv) | (~mk & mv);
    }
    char* st = As + stage * kAStageBytes;
    *reinterpret_cast<uint4*>(st + piece_offset(ra, q)) = make_uint4(plus[0], plus[1], plus[2], plus[3]);
    *reinterpret_cast<uint4*>(st + piece_offset(kTileRows + ra, q)) = make_uint4(minus[0], minus[1], minus[2], minus[3]);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // A fragments: row group i of a chunk lives in afr[i % 4] and is read from LDS two groups
  // before it is multiplied (row groups 0-1 of the next chunk at the end of the current one).
  bf16x8 afr[4];
  bf16x8 bq[kBRing][4];
  const int a_lane_off = piece_offset((kExact ? 0 : side * kTileRows) + (lane & 15), kp);
  auto read_a = [&](int stage, int i, bf16x8& dst) {
    // row group i: 16 * i rows further, i.e. 1024 * i bytes (the swizzle repeats every 16 rows)
    dst = *reinterpret_cast<const bf16x8*>(As + stage * kAStageBytes + a_lane_off + 1024 * i);
  };
  auto mma_group = [&](int i, const bf16x8& af, const bf16x8 (&b)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b[j], acc[i][j], 0, 0, 0);
  };
  // exact: W fragment in afr[2 (i % 2)], eps' P fragment (signs flipped for the -eps model) in
  // afr[2 (i % 2) + 1]; eps' P lies kTileRows rows (8 KB) after W, with the same swizzle
  const uint32_t pflip = side ? 0x80008000u : 0u;
  auto read_a2 = [&](int stage, int i, bf16x8& dw, bf16x8& dp) {
    const char* base = As + stage * kAStageBytes + a_lane_off + 1024 * i;
    dw = *reinterpret_cast<const bf16x8*>(base);
    dp = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + kTileRows * 64) ^ pflip);
  };
  // Activations of chunk c (clamped to the last one): fragment j is the 16 columns
  // 16 j .. 16 j + 15 of the wave, 512 elements further per fragment.
  auto load_b = [&](int c, bf16x8 (&d0)[4]) {
    const int c0 = min(c, nch - 1);
    const bool x0p = c0 < kx;
    const uint16_t* s0 = (x0p ? a.x_in : a.h_prev) + chunk_stride * (x0p ? c0 : c0 - kx);
#pragma unroll
    for (int j = 0; j < 4; ++j) d0[j] = *reinterpret_cast<const bf16x8*>(s0 + 16 * kKChunk * j + boff);
  };

  // One K step on chunk c (c % 4 == S). Requests go out at the top: on odd steps the weights of
  // chunks c+5 and c+6, then in every step the activations of chunk c+3 (one chunk per step
  // keeps the request stream even). Vector loads complete in issue order, and each
  // stream is consumed in issue order, so this order never makes a wait for one chunk hold up a
  // newer chunk: the weights of chunk c+5 are waited for in step c+1, after everything issued
  // before them was needed anyway. Row groups 0-5 are multiplied, each followed
  // by the fragment reads two groups ahead (row groups 2-7 of chunk c); chunk c+4 is selected
  // into its stage; row groups 6-7 finish, followed by the reads of row groups 0-1 of chunk c+1.
  // Selecting late in the step gives the weight requests more time to arrive. Past the last
  // chunk the requests repeat the last chunk and the select fills a stage that is never
  // multiplied (the phased instance leaves both out).
  //
  // The selected tiles live in an 8-stage ring (chunk k in stage k % 8), selected 4 chunks ahead,
  // and a barrier follows the select only in every fourth step (S = 3). That is enough:
  //  - the fragments of chunk c+1, selected in step c-3, are first read after row group 6 of
  //    step c, and one of steps c-3 .. c has its barrier between the two;
  //  - the select of chunk c+4 in step c overwrites the stage of chunk c-4, whose last reads
  //    (row group 7, after row group 5 of step c-4) complete before the barrier of whichever of
  //    steps c-4 .. c-1 has one.
  // Fewer barriers let the waves drift against each other and absorb memory latency.
  uint4 w_r[4];  // weight ring: chunk k in slot k % 4
  uint32_t wd_r[4];
  // Ph: kAll issues every request and select (clamped to the last chunk past the end); when the
  // chunk count is a multiple of 4 (and at least 8), the last two groups of four steps run as
  // kPenult and kLast, which leave out at compile time what would only repeat the last chunk:
  // kPenult the weight requests of its fourth step (chunks nch, nch + 1); kLast every weight
  // request and select, the activation requests of its last three steps (chunks nch and up) and
  // the fragment reads of chunk nch, and its barrier (it writes no LDS, and the selects of chunks
  // nch - 4 .. nch - 1 are followed by the barrier of kPenult's fourth step). The code stays
  // straight-line, so the compiler's waits count exactly the requests in flight.
  auto step = [&](int c, auto S, auto Ph) {
    constexpr int s_ = decltype(S)::value;
    constexpr int ph = decltype(Ph)::value;
    constexpr int wuse = s_;
    constexpr bool w_req = s_ % 2 == 1 && ph != kLast && !(ph == kPenult && s_ == 3);
    constexpr bool b_req = ph != kLast || s_ == 0;
    constexpr bool sel = ph != kLast;
    constexpr bool next_reads = !(ph == kLast && s_ == 3);
    const int rs = c & (kAStages - 1), rs1 = (c + 1) & (kAStages - 1), ws = (c + 4) & (kAStages - 1);
    if constexpr (w_req) {
      load_w(min(c + 5, nch - 1), w_r[(s_ + 1) % 4], wd_r[(s_ + 1) % 4]);
      load_w(min(c + 6, nch - 1), w_r[(s_ + 2) % 4], wd_r[(s_ + 2) % 4]);
    }
    if constexpr (b_req) load_b(c + 3, bq[(s_ + 3) % 4]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (kExact) {
        const int cur = 2 * (i % 2), nxt = 2 * ((i + 1) % 2);
        mma_group(i, afr[cur], bq[s_]);
        mma_group(i, afr[cur + 1], bq[s_]);
        if (i + 1 < 8) read_a2(rs, i + 1, afr[nxt], afr[nxt + 1]);
        else if constexpr (next_reads) read_a2(rs1, 0, afr[nxt], afr[nxt + 1]);
      } else {
        mma_group(i, afr[i % 4], bq[s_]);
        if (i + 2 < 8) read_a(rs, i + 2, afr[(i + 2) % 4]);
        else if constexpr (next_reads) read_a(rs1, i - 6, afr[(i + 2) % 4]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (i == 5) {
        if constexpr (sel) {
          form_w(w_r[wuse], wd_r[wuse], ws);
          if constexpr (s_ == 3) __syncthreads();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Gate biases of both models for the tile's 32 units, [model][gate][unit], into LDS.
  float* bias_s = reinterpret_cast<float*>(As + kGateBiasOffset);
  if (tid < 2 * 4 * kUnitsPerTile) {
    const int sd = tid >> 7, g = (tid >> 5) & 3, u = tid & 31;
    bias_s[tid] = a.bias_m[(static_cast<int64_t>(2 * pr + sd) * a.L + a.layer) * (4 * H) + g * H + u0 + u];
  }

  // Prologue: activations of chunks 0-2 and weights of chunks 0-5 requested, chunks 0-3
  // selected into stages 0-3, row groups 0-1 of chunk 0 read.
  {
    uint4 wp[4];
    uint32_t dp[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) load_w(min(k, nch - 1), wp[k], dp[k]);
    load_w(min(4, nch - 1), w_r[0], wd_r[0]);
    load_w(min(5, nch - 1), w_r[1], wd_r[1]);
    load_b(0, bq[0]);
    load_b(1, bq[1]);
    load_b(2, bq[2]);
#pragma unroll
    for (int k = 0; k < 4; ++k) form_w(wp[k], dp[k], k);
  }
  __syncthreads();
  if constexpr (kExact) {
    read_a2(0, 0, afr[0], afr[1]);
  } else {
    read_a(0, 0, afr[0]);
    read_a(0, 1, afr[1]);
  }

  static_assert(kBRing == 4, "the step is unrolled for a ring of 4");
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  auto group = [&](int c0, auto Ph) {
    step(c0, S0{}, Ph);
    step(c0 + 1, S1{}, Ph);
    step(c0 + 2, S2{}, Ph);
    step(c0 + 3, S3{}, Ph);
  };
  // This lane's cell state: tile-private, stored in accumulator order, so each row group is one
  // 16-byte access per lane and 1 KB per wave. It is read and written once per launch by this
  // workgroup alone: its accesses (and the h stores) are marked non-temporal, which keeps them
  // from displacing the weight and activation lines that the workgroups of an XCD share in L2
  // (charlm launch -1.5 to -2.2%). The phased instance requests it early, into the activation
  // registers its last steps no longer fill: row groups 0-3 into those of chunk nch - 4 before the
  // second of the last four steps, 4-7 into those of chunk nch - 3 before the third (at the first
  // timestep it reads whatever the buffer holds, in bounds, and uses zeros). A generic lambda, so
  // that only the phased instance instantiates it.
  auto c_early = [&](auto& dst, auto I0) {
    constexpr int i0 = decltype(I0)::value;
    const int64_t tile = (static_cast<int64_t>(pr) * a.n_col_blocks + cb) * a.n_row_tiles + rt;
    const f32x4* cp = reinterpret_cast<const f32x4*>(a.c_tile) + (tile * 8 + wave) * 8 * 64 + lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(cp + 64 * (i0 + i)));
  };
  using All = std::integral_constant<int, kAll>;
  int c = 0;
  if constexpr (kPhased) {
    // every request of a group starting at c is for a chunk below nch while c + 12 <= nch
    for (; c + 12 <= nch; c += 4) group(c, All{});
    group(c, std::integral_constant<int, kPenult>{});
    using Last = std::integral_constant<int, kLast>;
    step(c + 4, S0{}, Last{});
    c_early(bq[0], std::integral_constant<int, 0>{});
    step(c + 5, S1{}, Last{});
    c_early(bq[1], std::integral_constant<int, 4>{});
    step(c + 6, S2{}, Last{});
    step(c + 7, S3{}, Last{});
  } else {
    for (; c + 4 <= nch; c += 4) {
      step(c, S0{}, All{});
      step(c + 1, S1{}, All{});
      step(c + 2, S2{}, All{});
      step(c + 3, S3{}, All{});
    }
    if (c < nch) step(c, S0{}, All{});
    if (c + 1 < nch) step(c + 1, S1{}, All{});
    if (c + 2 < nch) step(c + 2, S2{}, All{});
  }

  const int64_t tile = (static_cast<int64_t>(pr) * a.n_col_blocks + cb) * a.n_row_tiles + rt;
  float4* cptr = reinterpret_cast<float4*>(a.c_tile) + (tile * 8 + wave) * 8 * 64 + lane;
  f32x4 cst[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (kPhased)
      cst[i] = a.first ? f32x4{0.f, 0.f, 0.f, 0.f} : __builtin_bit_cast(f32x4, bq[i >> 2][i & 3]);
    else
      cst[i] = a.first ? f32x4{0.f, 0.f, 0.f, 0.f} : __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(cptr + 64 * i));
  }
  // ---- fused LSTM cell; h leaves from registers as whole 64-byte column segments -------------
  // Lane (row r = lane / 16, column lane % 16 of each 16-column block j) holds unit 4 i + r of row
  // group i. The bf16 h of row groups 2k and 2k + 1 share a register (units 8k + r and 8k + 4 + r),
  // the four registers of a column block are exchanged among the four rows (row_exchange), and a
  // byte permute re-pairs them so that row r holds units 8r .. 8r + 7: one 16-byte store per lane
  // and column block, 1 KB of contiguous h per store instruction, without LDS or a barrier.
  uint32_t hd[4][4];  // [j][k]: bf16 h of units 8k + r (low half) and 8k + 4 + r (high half)
  float hprev[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ul = 4 * i + (lane >> 4);
    const float* bs = bias_s + side * 4 * kUnitsPerTile + ul;
    const float bi = bs[0], bf = bs[kUnitsPerTile], bg = bs[2 * kUnitsPerTile], bo = bs[3 * kUnitsPerTile];
    const float cprev[4] = {cst[i][0], cst[i][1], cst[i][2], cst[i][3]};
    float cn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float hv;
      lstm_cell(acc[i][j][0] + bi, acc[i][j][1] + bf, acc[i][j][2] + bg, acc[i][j][3] + bo, cprev[j], cn[j], hv);
      if (i & 1) {
        // hardware round-to-nearest-even conversion (equal to f32_to_bf16_rne except for NaN payloads)
        const f32x2 hp = {hprev[j], hv};
        hd[j][i >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hp, bf16x2));
      } else {
        hprev[j] = hv;
      }
    }
    __builtin_nontemporal_store(f32x4{cn[0], cn[1], cn[2], cn[3]}, reinterpret_cast<f32x4*>(cptr + 64 * i));
  }
  const int hrow = lane >> 4;
  const int64_t hcol0 = static_cast<int64_t>(2 * pr + side) * a.B;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // afterwards hd[j][x] holds units 8 hrow + x (low half) and 8 hrow + 4 + x (high half)
    row_exchange(hd[j][0], hd[j][1], hd[j][2], hd[j][3]);
    const uint4 out = make_uint4(__builtin_amdgcn_perm(hd[j][1], hd[j][0], 0x05040100u),
                                 __builtin_amdgcn_perm(hd[j][3], hd[j][2], 0x05040100u),
                                 __builtin_amdgcn_perm(hd[j][1], hd[j][0], 0x07060302u),
                                 __builtin_amdgcn_perm(hd[j][3], hd[j][2], 0x07060302u));
    const int b = bcol0 + 64 * cq + 16 * j + (lane & 15);
    if (b < a.B) {
      uint16_t* dst = a.h_out + (static_cast<int64_t>(rt) * a.ncols_pad + hcol0 + b) * kKChunk + 8 * hrow;
      __builtin_nontemporal_store(u32x4{out.x, out.y, out.z, out.w}, reinterpret_cast<u32x4*>(dst));
    }
  }
}

}  // namespace cdrge
