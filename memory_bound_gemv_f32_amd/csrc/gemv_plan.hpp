// Host-side mapping of a GEMV problem onto gfx950 workgroups.
//
// Pure C++ (no HIP headers): the same function decides what the entry points
// launch and what gemv_plan() reports, so the mapping table can be checked on
// a machine without a GPU.
//
// The one design axis is how many lanes cooperate on one row's dot product
// (page "SGEMV CUDA代码学习", section "三 kernel 的设计空间总结": elements per
// lane times rows per warp equals the warp width, so that no lane idles).  On
// a 64-lane wavefront with 16-byte loads, one load instruction covers 1 KiB
// of A, so:
//   * rows shorter than 32 loads (fp32 K <= 128, fp16/bf16 K <= 256) share a
//     wavefront: L lanes per row, L the next power of two of the row's load
//     count, 64/L rows per wavefront (the page's section "Kernel 3: k16", two
//     rows per warp, generalised);
//   * mid-length rows get one wavefront each (its sections "Kernel 1: k32"
//     and "Kernel 2: k128 + Vec4");
//   * long rows when there are too few rows to fill the chip get a whole
//     workgroup each with a cross-wavefront reduction in LDS (page "第 3 课：
//     GEMV 与行级并行", section "2. 行级并行与 Block 映射架构" and the
//     threshold discussion of its section "4. 性能与工程权舍").
// The thresholds are this library's own, set for 256 CUs.
#pragma once

#include <stdint.h>

namespace gemvplan {

enum Dtype { F32 = 0, F16 = 1, BF16 = 2 };
// Int8 weights: planned by their own 1-byte rows (16 weights per load); x
// keeps its float type (validate_q8).
constexpr int Q8 = 3;
enum Family {
    AUTO = -1,
    ROWS_PER_WAVE = 0,
    WAVE_PER_ROW = 1,
    GROUP_PER_ROW = 2,
    BATCHED = 3,
    BATCHED_MFMA = 4,
    GATED_SILU = 5,
    SPLIT_K = 6
};
enum Status { OK = 0, INVALID = 1 };

constexpr int kWave = 64;
constexpr int kLoadBytes = 16;
// Right-hand vectors of the batched entry points.  The vector-ALU batched
// kernel keeps one accumulator per (row, vector) in registers and takes at
// most kValuVectors per launch; the matrix-core kernel takes up to
// kMaxVectors in one pass over A (tiles of 16 vectors).
constexpr int kMaxVectors = 64;
constexpr int kValuVectors = 16;

// Rows-per-wave family: lanes per row is a power of two up to this.
constexpr int kRowsPerWaveMaxLanes = 32;
// Workgroup-per-row family: wavefronts per workgroup, and when it is chosen
// automatically: few rows (fewer than there are CUs' worth of wavefronts),
// long rows (a wavefront per row would walk them in several dependent
// batches), or very many rows.
// (Many rows: from 6144 rows of 512 loads the workgroup per row was ahead,
// bf16 × 4096, µs, wavefront / workgroup per row: 4096 rows 6.60 / 6.70,
// 6144 8.86 / 8.80, 7168 10.10 / 9.93, 8192 10.93 / 10.89; the fused q/k/v
// call over 6144 rows 9.08 / 8.87.)
constexpr int kGroupWaves = 4;
// Few long rows: below kGroupWideMaxRows rows, workgroups of 4 wavefronts
// keep too few bytes in flight when each lane needs more than one batch of
// loads; then a workgroup of one row has kGroupWideWaves wavefronts and one
// of two rows kGroupWidePairWaves.  MI355X, µs with 4 -> 8 -> 16 wavefronts:
// one row, bf16 192 × 65536 7.77, 7.33, 6.94; bf16 256 × 65536 8.14, 7.64,
// 7.38; fp32 256 × 32768 8.06, 7.54, 7.37; bf16 384 × 32768 7.20, 6.88,
// 6.87; two rows, bf16 512 × 32768 7.28, 6.92, 7.23; fp16 1000 × 20000
// 8.29, 8.01, 8.26; bf16 900 × 30000 11.13, 10.78, 11.00.
constexpr int kGroupWideWaves = 16;
constexpr int kGroupWidePairWaves = 8;
constexpr int64_t kGroupWideMaxRows = 1024;
constexpr int64_t kGroupMaxRows = 256;
// Rows of at least kGroupMidMinLoads loads (every lane of a workgroup busy)
// take a workgroup each up to kGroupMidRows rows.  MI355X, bf16, µs, wave /
// workgroup per row: 384 × 4096 2.86 / 2.62, 512 × 4096 2.88 / 2.73, 640 ×
// 4096 2.99 / 2.93, 768 × 4096 3.03 / 3.05, 896 × 4096 3.12 / 3.24, 1024 ×
// 4096 3.20 / 3.37; 384 × 2048 2.37 / 2.30, 640 × 2048 2.48 / 2.47, 768 ×
// 2048 2.55 / 2.54, 896 × 2048 2.62 / 2.63.
constexpr int64_t kGroupMidRows = 704;
constexpr int64_t kGroupMidMinLoads = 256;
constexpr int64_t kGroupLongRowLoads = 1024;
constexpr int64_t kGroupManyRows = 6144;
constexpr int64_t kGroupManyRowsMinLoads = 512;
// Wave-per-row family: loads per lane kept in flight per row.
constexpr int kWaveBatch = 8;
constexpr int kGroupBatch = 8;
// Workgroup-per-row family: when x is longer than kGroupShareMinXBytes (it
// no longer stays in a CU's vector L1 next to the A stream, and a workgroup
// per row would fetch all of x from L2 once per row), up to
// kGroupMaxTileRows rows per workgroup share each x chunk, as long as rows ×
// loads per lane stays within kGroupTileLoads per batch and at least
// kGroupTileMinGroups workgroups remain.  Measured on MI355X, bf16
// 4096 × 14336: 21.7 -> 20.1 µs with two rows per workgroup; with an 8 KiB x
// (4096 × 4096, 14336 × 4096) sharing it was 1-9 % slower.
constexpr int64_t kGroupShareMinXBytes = 16 * 1024;
constexpr int kGroupMaxTileRows = 2;
constexpr int kGroupTileLoads = 16;
constexpr int64_t kGroupTileMinGroups = 256;
// When x is longer than kGroupStreamMinXBytes and at most
// kGroupStreamMaxChunks 16-byte chunks per lane (8 KiB < x <= 24 KiB: bf16
// 4096 < K <= 12288, fp32 2048 < K <= 6144) and K is whole chunks, each lane
// keeps its x chunks in registers and the workgroup walks up to
// kGroupStreamRows rows (halved while fewer than kGroupTileMinGroups
// workgroups would remain), each row's loads issued before the previous
// row's multiply-adds; such shapes take this family even where a wavefront
// per row would otherwise run them.  Measured on MI355X (bf16, µs, before ->
// after): 4096 × 6144 9.97 -> 8.95, 4096 × 8192 12.2 -> 11.4, 8192 × 8192
// 22.0 -> 20.5, 2048 × 8192 7.41 -> 6.85; 4096 × 10240 15.2 (two rows per
// workgroup) -> 13.5.  At 7 chunks (bf16 4096 × 14336) two rows per
// workgroup were faster (18.1 against 18.4 µs on three boxes), and with an
// 8 KiB x (4096 × 4096, 14336 × 4096) the wavefront and workgroup per row
// were (6.60 against 6.70, 17.4 against 17.5).
constexpr int64_t kGroupStreamMinXBytes = 8 * 1024;
constexpr int kGroupStreamWaves = 4;
constexpr int kGroupStreamMaxChunks = 6;
constexpr int kGroupStreamRows = 4;
constexpr int kQ8StreamMaxChunks = 4;
constexpr int kQ8StreamMaxChunksWideX = 3;
// Compute units of the GPU this library is built for (MI355X).
constexpr int64_t kCUs = 256;
// Batched family on the vector ALUs (a wavefront per group of rows, all
// vectors at once): rows per wavefront (they share every X chunk), loads of
// A per lane per batch, and whether a batch's X chunks are loaded with its A
// chunks (few vectors) or chunk by chunk after them (many: their X chunks
// would not fit the registers), chosen so that the loaded chunks, the
// accumulators and the compensated sums fit two wavefronts per SIMD.
// Two rows per wavefront once the grid of 2-row workgroups (4 wavefronts,
// 8 rows) covers every compute unit at least twice, or more than once with
// 4 or more vectors; else one, whose grid of twice as many workgroups keeps
// more wavefronts in flight.  fp16, K = 4100 (the unaligned rows this
// family serves), µs, one row / two: 1024 rows, 2 vectors 3.87 / 5.02 and
// 16 vectors 10.93 / 15.66; 2048 rows, 4 vectors 6.45 / 8.05; 3072 rows,
// 2 vectors 6.76 / 7.68 and 8 vectors 15.00 / 13.47; 4096 rows, 4 vectors
// 11.34 / 9.14 and 16 vectors 30.20 / 24.24; 8192 rows, 2 vectors 14.61 /
// 13.13 and 16 vectors 57.30 / 44.11.
constexpr int batched_rows(int64_t M, int nvec) {
    const int64_t groups = (M + 7) / 8;
    return groups >= 2 * kCUs || (groups > kCUs && nvec >= 4) ? 2 : 1;
}
constexpr int batched_batch(int nvec) { return nvec <= 2 ? 4 : 2; }
constexpr bool batched_x_ahead(int nvec) { return nvec <= 8; }
// Batches whose products run into one accumulator before it is added to
// the compensated sum.  Past 8 vectors (X loaded chunk by chunk) the kernel
// is bound by its vector-ALU work, and the compensated add of each (row,
// vector) costs nearly as much as the batch's 16 multiply-adds: there an
// accumulator runs over kBatchedRunElems elements per lane (a batch of B
// chunks of E elements covers B·E) and the multiply-adds of all (row,
// vector) pairs are interleaved word by word.  fp16 K = 4100, 16 vectors,
// µs, one batch per run / runs of 64 elements: 512 rows 10.58 / 8.99, 3072
// 23.62 / 21.72, 4096 24.22 / 22.36, 8192 44.07 / 40.58; bf16 1024 rows
// 13.13 / 10.65.  Up to 8 vectors the same form changed times by -12 to +8 %
// from shape to shape (mostly slower), so there every batch is added.
constexpr int kBatchedRunElems = 64;
constexpr int batched_run(int nvec, int batch, int chunk_elems) {
    return batched_x_ahead(nvec) || batch * chunk_elems >= kBatchedRunElems
               ? 1
               : kBatchedRunElems / (batch * chunk_elems);
}
// Wavefronts per row: with one row per wavefront the time is one
// wavefront's walk along its row, and few rows leave most of the chip idle.
// Up to kBatchedSplitMaxRows rows (one wavefront on at most every other
// SIMD) the workgroup's 4 wavefronts share each row (every fourth batch
// each, totals added in LDS).  fp16, µs, one row per wavefront / per
// workgroup: K = 4100, 64 rows 2 vectors 3.43 / 2.63, 16 vectors 8.96 /
// 5.47; 512 rows 2 vectors 3.69 / 3.32, 8 vectors 7.72 / 5.04, 16 vectors
// 9.12 / 7.50; 64 × 14337 16 vectors 40.21 / 13.51; 512 × 11009 16 vectors
// 33.05 / 19.40; at 1024 rows mixed (8 vectors 7.91 / 7.06, 16 vectors 9.48
// / 12.19), from 1536 rows slower (2048 rows 16 vectors 16.27 / 21.25).
// Up to kBatchedPairMaxRows rows with at least kBatchedPairMinVectors
// vectors, pairs of wavefronts share each row instead (K = 4100, µs, one /
// two wavefronts per row: 600 rows 4 vectors 5.49 / 4.48, 8 vectors 7.77 /
// 6.89; 1024 rows 4 vectors 5.62 / 4.68, 16 vectors 9.46 / 9.56; 1536 rows
// 8 vectors 10.46 / 8.89, 16 vectors 15.93 / 13.88; bf16 1024 rows 8
// vectors 8.67 / 6.81); with 2 vectors pairs lost 1-4 % (1024 rows 3.89 /
// 4.03), and at 2048 rows 3-8 % (4 vectors 6.42 / 6.89).
constexpr int64_t kBatchedSplitMaxRows = 512;
constexpr int kBatchedSplit = 4;
constexpr int64_t kBatchedPairMaxRows = 1536;
constexpr int kBatchedPairMinVectors = 4;
constexpr int batched_split(int64_t M, int nvec) {
    if (M <= kBatchedSplitMaxRows) return kBatchedSplit;
    return M <= kBatchedPairMaxRows && nvec >= kBatchedPairMinVectors ? 2 : 1;
}
// Matrix-core batched family: up to kMfmaRows rows per workgroup (4, 8, 16
// or 32, below), its wavefronts split K and walk their slice in chunks of
// this many 64-wide steps (the A loads of a chunk are in flight together;
// X's chunk is staged in LDS).
constexpr int kMfmaRows = 32;
constexpr int kMfmaWaves = 8;
constexpr int kMfmaChunk = 8;
// Up to this many vectors the matrix-core kernel reads its X operands
// straight from memory (a load touches only the columns in use) instead of
// staging X in LDS (fp16 4096 × 4096, µs, straight / staged: 3 vectors
// 7.07 / 7.15, 4 7.19 / 7.25, 5 7.25 / 7.27, 6 7.38 / 7.30, 8 7.63 / 7.38).
constexpr int kMfmaFewVectors = 5;
// With more 16-row tiles than compute units, workgroups of
// kMfmaManyTilesWaves wavefronts (each walking two chunks of its longer K
// run, half the LDS): two fit on a compute unit, so one's loads overlap the
// other's tail, where a workgroup of 8 (130 KiB of LDS) runs alone, start to
// finish.  MI355X, fp16 K = 4096, µs, 8 / 4 wavefronts, 4 and 16 vectors:
// 6144 rows 11.96 / 11.68 and 13.63 / 13.08, 8192 13.11 / 12.63 and 14.39 /
// 13.73, 14336 23.49 / 21.03 and 26.50 / 24.16, 28672 41.53 / 36.90 and
// 46.71 / 41.64; at one tile per unit or fewer 8 stays (4096 7.24 / 8.05 and
// 7.87 / 8.50, 1024 6.04 / 6.66).  (2 wavefronts: 14336 22.2 and 23.7,
// 28672 42.8 and 47.5.)
constexpr int kMfmaManyTilesWaves = 4;
// Groups of 8 real rows per matrix-core workgroup: one while 8-row
// workgroups fill the compute units at most once (M <= 2048), else two.
// fp16 K = 4096, µs, two groups / one, 4 and 16 vectors: 1024 rows 6.04 /
// 4.89 and 7.02 / 5.75, 2048 6.21 / 5.17 and 7.23 / 6.04; 3072 (one group in
// 384 workgroups of 4 wavefronts) 6.66 / 8.04 and 7.64 / 9.63.
//
// Four groups (32 rows, half-size chunks) for kMfmaTallMinVectors (6) to 16
// vectors on tall matrices: every workgroup stages the whole of X for its
// rows, so 32-row workgroups read half as many X bytes per A byte.  The
// time of these grids follows the largest number of workgroups a compute
// unit runs, times their rows: four groups are taken when their grid has
// more workgroups than compute units (so 4 wavefronts each) and no unit runs
// more rows than with two.  fp16 K = 4096, µs, two groups / four: 16 vectors
// 12288 rows 19.49 / 21.24 (3 against 2·2 units of 16 rows), 13312 23.75 /
// 21.27, 14336 24.17 / 21.68, 16384 24.89 / 23.04, 20480 30.50 / 30.34 (5
// against 6); 9 vectors 13312 21.62 / 20.40, 16384 22.97 / 22.68, 28672
// 37.62 / 38.25 (7 against 8); 6-8 vectors gained less (13312 rows 6
// vectors 20.93 / 20.14, 8 vectors 21.32 / 20.31; 14336 rows 6 vectors
// 21.27 / 20.69; bf16 14336 rows 8 vectors 21.73 / 20.82; 16384 rows, both
// grids even, 6 vectors 22.34 / 22.61, 8 vectors 22.77 / 22.66).  With 8
// wavefronts (at most one workgroup per unit) four groups were slower: 4096
// rows 7.84 / 11.30, 8192 13.79 / 15.90.  (Up to kMfmaFewVectors vectors X
// is read straight from memory and the kernel takes at most two groups.)
constexpr int kMfmaTallMinVectors = kMfmaFewVectors + 1;
constexpr int mfma_row_groups(int64_t M, int nvec) {
    if ((M + 7) / 8 <= kCUs) return 1;
    const int64_t g2 = (M + 15) / 16, g4 = (M + 31) / 32;
    const bool four = nvec >= kMfmaTallMinVectors && nvec <= 16 && g4 > kCUs &&
                      2 * ((g4 + kCUs - 1) / kCUs) <= (g2 + kCUs - 1) / kCUs;
    return four ? 4 : 2;
}
// Real rows per group: 8, or, with X staged in LDS (more than
// kMfmaFewVectors vectors), 4 (one group) while 4-row workgroups fill the
// compute units at most once (M <= 1024).  fp16 K = 4096, µs, 8 / 4 rows per
// workgroup: 16 vectors 256 rows 5.53 / 5.01, 1024 rows 5.75 / 5.29; 33
// vectors 1024 rows 10.18 / 10.09; with X read straight from memory 4 rows
// gained nothing (2 vectors 4.73 / 4.75, 4 vectors 4.89 / 4.95 at 1024 rows).
constexpr int mfma_group_rows(int64_t M, int nvec) {
    return nvec > kMfmaFewVectors && (M + 3) / 4 <= kCUs ? 4 : 8;
}
constexpr int mfma_waves(int64_t M, int rows_per_group) {
    return (M + rows_per_group - 1) / rows_per_group > kCUs ? kMfmaManyTilesWaves : kMfmaWaves;
}
// 16-vector tiles for nvec vectors (1, 2 or 4); the chunk shrinks as the
// tiles grow so that the X staged per chunk stays 16 KiB per wavefront, and
// is halved with four row groups (twice the A loads per step: the chunk's
// A, X and accumulators then fit the registers of two wavefronts per SIMD).
constexpr int mfma_tiles(int nvec) { return nvec <= 16 ? 1 : (nvec <= 32 ? 2 : 4); }
constexpr int mfma_chunk(int nvec, int groups = 2) {
    return kMfmaChunk / mfma_tiles(nvec) / (groups == 4 ? 2 : 1);
}
constexpr int mfma_lds_bytes(int nvec, int waves, int groups = 2) {
    return waves * 16 * mfma_tiles(nvec) * (mfma_chunk(nvec, groups) * 128 + 16);
}
// The 64-element steps of a row that wavefront `wave` of a matrix-core
// workgroup of `waves` wavefronts walks: steps [first, end) of the
// ceil(K/64) steps, the last of which may be partial (K % 64 != 0).  The
// steps are dealt in contiguous runs of ceil(steps/waves); trailing
// wavefronts may get an empty run.  Every step, the partial one included,
// belongs to exactly one wavefront.  (A constexpr function: the kernel calls
// it on the device, the host tests call it on the CPU.)
struct StepRange {
    int first;
    int end;
};
constexpr StepRange mfma_step_range(int K, int waves, int wave) {
    const int steps = K / 64 + (K % 64 != 0 ? 1 : 0);
    const int per = (steps + waves - 1) / waves;
    const int first = wave * per < steps ? wave * per : steps;
    const int end = first + per < steps ? first + per : steps;
    return StepRange{first, end};
}

// ---- rounding-chain bound --------------------------------------------------
//
// Every output is a sum of K exact products (fp16/bf16 products are exact in
// fp32; fp32 products are fused into FMAs) formed through a tree of fp32
// additions.  If no product passes through more than n roundings on its way
// to the output, |y - exact| <= γ_n·Σ_k|A[m,k]·x[k]|, γ_n = n·u/(1 - n·u),
// u = 2^-24: n <= 167 keeps every output within 1e-5·Σ|A·x| for every input,
// not only for inputs whose rounding errors happen to cancel.  (Page "GEMM、
// GEMV、dtype 与算术强度", section "dtype 改变什么": the accumulator is where
// precision is kept.)  rounding_chain() gives n for a plan; the planner keeps
// it within kMaxRoundingChain.
constexpr int kMaxRoundingChain = 150;
// v_dot2_f32_{f16,bf16}: two exact products and the accumulator passed in,
// aligned to the largest of the three with the bits more than about 24
// places below it dropped, then rounded once (measured on gfx950: with
// 2^k, -2^k and an accumulator of 1 the 1 survives up to k = 24; 2^23 +
// 0.75 gives 2^23).  Each term can lose less than 2^-23 of the largest:
// charged 3·2 + 1 = 7 roundings of the running sum per instruction.
constexpr int kDot2Roundings = 7;
// One 16×16×32 matrix-core step from a zero accumulator: the matrix core
// aligns an output's 32 products to the largest and keeps about 24 bits
// below it (measured on gfx950: 2^k + 1 - 2^k gives 1 for k <= 24, 0 from
// k = 25), dropping the rest, then rounds once to fp32.  Each product can
// lose less than 2^-23 of the largest, so the step's error is below
// (32·2 + 1)·u·Σ|products|: charged as 65 roundings.  The kernel adds each
// step's outputs to its accumulators with fp32 additions (one rounding per
// step), never passing a running sum into the matrix core.
constexpr int kMfmaProductRoundings = 65;

inline int ceil_log2(int64_t v) {
    int r = 0;
    while (((int64_t)1 << r) < v) ++r;
    return r;
}

// Roundings a compensated (error-free two-sum) running sum of n terms adds:
// its result is within u·|sum| + γ_{n-1}²·Σ|terms| (Ogita, Rump and Oishi,
// "Accurate sum and dot product", algorithm Sum2): one rounding plus
// γ_{n-1}²/u.  One term is exact.
inline int compensated_roundings(int64_t n) {
    if (n <= 1) return 0;
    const double u = 1.0 / 16777216.0;
    const double g = (double)(n - 1) * u / (1.0 - (double)(n - 1) * u);
    const double extra = g * g / u;
    return 1 + (int)(extra + 0.999999);
}

// The vector-ALU bodies (rows per wavefront, wave per row, workgroup per
// row, gated, split-K pass 1): `elems` elements per row (or slice), chunks
// of `chunk` elements, `lanes` lanes per row of which `wave_lanes` share a
// wavefront, `batch` chunks per lane per batch summed into two fresh
// accumulators (alternate chunks), the batches' sums (and the sum of the
// element-wise tail) added with a compensated running sum, then a tree over
// the wavefront's lanes and a sequential fold of `waves` wavefronts' partials.
// `per_elem` roundings per element within an accumulator (1 for FMA).
// `accs` accumulators take the chunks of a batch in turn (2, or 1 in the
// vector-ALU batched kernel).
inline int valu_chain(int64_t elems, int chunk, int lanes, int wave_lanes, int batch, int waves,
                      int per_elem = 1, int accs = 2) {
    const int64_t full = elems / chunk;
    const int64_t tail = elems - full * chunk;
    const int64_t per_lane = (full + lanes - 1) / lanes;
    const int64_t b = per_lane < batch ? (per_lane < 1 ? 1 : per_lane) : batch;
    const int64_t batches = (per_lane + batch - 1) / batch;
    const int64_t in_batch = (b + accs - 1) / accs * chunk * per_elem + (accs - 1);
    const int64_t in_tail = (tail + lanes - 1) / lanes;
    const int64_t first = in_batch > in_tail ? in_batch : in_tail;
    const int64_t terms = batches + (tail > 0 ? 1 : 0);
    return (int)(first + compensated_roundings(terms) + ceil_log2(wave_lanes) + (waves - 1));
}

// The vector-ALU batched kernel: rows of `elems` elements in chunks of
// `chunk`, batches of `batch` chunks per lane (64 lanes per wavefront), a
// wavefront taking every `split`-th batch; runs of up to `run` batches
// accumulate in place before a compensated add (the element-wise tail is
// one more term); then the 64-lane tree and the in-order fold of the split
// wavefronts' totals.
inline int batched_chain(int64_t elems, int chunk, int batch, int run, int split) {
    const int64_t full = elems / chunk;
    const int64_t tail = elems - full * chunk;
    const int64_t per_block = (int64_t)batch * 64;
    const int64_t blocks = (full + per_block - 1) / per_block;
    const int64_t mine = (blocks + split - 1) / split;  // batches of the busiest wavefront
    const int64_t in_run = (mine < run ? mine : run) * batch * chunk;
    const int64_t in_tail = (tail + 63) / 64;
    const int64_t terms = (mine + run - 1) / run + (tail > 0 ? 1 : 0);
    return (int)((in_run > in_tail ? in_run : in_tail) + compensated_roundings(terms) + ceil_log2(64) +
                 (split - 1));
}

// The matrix-core kernel: each wavefront's run of 64-wide steps in chunks of
// `ch` steps; with `fresh` every chunk (and the leftover steps) sums into
// fresh accumulators added with a compensated running sum, otherwise all
// steps accumulate in place.  Then the two half-row tiles are added and the
// `waves` wavefronts' partial tiles folded in order.
inline int mfma_chain(int K, int waves, int ch, bool fresh) {
    const int steps = mfma_step_range(K, waves, 0).end;  // the longest run
    if (!fresh) return kMfmaProductRoundings + steps + 1 + (waves - 1);
    const int chunks = steps / ch + (steps % ch != 0 ? 1 : 0);
    return kMfmaProductRoundings + ch + compensated_roundings(chunks) + 1 + (waves - 1);
}
// Split-K: when there are too few rows to fill the chip and each row holds
// much more than a workgroup keeps in flight (page "SGEMV CUDA代码学习",
// section "Kernel 1: k32": with M = 8 only two blocks run and the rest of the
// machine idles), every row is cut into `splits` slices; a workgroup per
// (pair of rows, slice) writes the two rows' partial sums, and a second
// kernel adds each row's partials in slice order (a fixed order, so results
// are reproducible).  Two rows per workgroup let each x chunk serve both
// (a workgroup otherwise reads as many x bytes as A bytes); four were
// slower.  MI355X, µs with 1 -> 2 rows per workgroup, reduce included: fp32
// 8×2^21 15.49 -> 14.59, bf16 64×2^18 9.21 -> 8.77, fp16 32×2^19 9.34 ->
// 8.62, fp32 100×2^18 23.87 -> 20.92, bf16 7×2^20 6.64 -> 6.26; with 4
// rows 15.06, 9.55, 9.32, 21.70, 7.79 (and no better with 2-4x the slices).
// Chosen automatically for fewer than kSplitMaxRows rows of at least
// kSplitMinRowLoads 16-byte loads (4 batches of the workgroup-per-row
// family); below that the second launch (~2 µs) costs more than it saves.
// Slices are at least kSplitMinSliceLoads loads, a whole number of 64-lane
// loads, and their count a multiple of 8 when it is 8 or more (see the
// pass-1 kernel: then every XCD serves whole slices of x).  Measured on
// MI355X, the reduce launch included: fp32 8×2^21 265 -> 15.6 µs, fp32
// 1×2^24 2147 -> 24.4 µs, bf16 64×2^18 20.7 -> 9.3 µs, bf16 128×2^17
// 12.26 -> 8.47 µs; but unsplit is faster from about 200 rows up (bf16
// 200×2^16 7.81 against 8.05 split, 255×2^16 8.12 against 8.46, fp32
// 255×2^15 8.03 against 8.43; 256×2^16 and 512×2^15 likewise).
constexpr int64_t kSplitMaxRows = 192;
constexpr int64_t kSplitMinRowLoads = 4 * kGroupWaves * kWave * kGroupBatch;
constexpr int64_t kSplitMinSliceLoads = 512;
constexpr int kSplitMaxSplits = 1024;
constexpr int kSplitRowsPerGroup = 2;
// Int8 weights: loads per lane per batch (each weight chunk brings a 32- or
// 64-byte x chunk), and the workgroups below which a wavefront keeps one
// row instead of two.
constexpr int kQ8Batch = 4;
constexpr int64_t kQ8PairRowsMinGroups = 256;
// Int8 rows of at least kGroupMidMinLoads loads run the workgroup-per-row
// family up to kQ8GroupMaxRows rows.  Up to kQ8OneRowMaxRows rows with an
// x row under kQ8PairMinXBytes a workgroup takes one row; otherwise two,
// which share every x chunk, while at least kQ8PairMinGroups workgroups
// remain.  MI355X, µs, wave per row (two rows per wavefront) / workgroup of
// one row / of two rows / of four: int8 4096 × 4096 with fp16 x 5.08 /
// 4.76 / 4.90 / 5.15, with fp32 x - / 6.24 / 5.46 / 5.40; 4096 × 11008 fp16
// x - / 11.34 / 9.64 / 9.62; 2048 × 8192 fp16 x - / 5.20 / 5.21 / 5.58;
// 11008 × 4096 fp16 x 9.40 / 9.27 / 8.47 / 9.06; 14336 × 4096 bf16 x 10.52
// / 11.74 / 10.42 / 10.89; wave per row / workgroup of two rows: 16384 ×
// 4096 fp16 x 12.07 / 11.28, 28672 × 4096 bf16 x 18.19 / 18.82.
constexpr int64_t kQ8GroupMaxRows = 16384;
constexpr int64_t kQ8OneRowMaxRows = 4096;
constexpr int64_t kQ8PairMinXBytes = 16 * 1024;
constexpr int64_t kQ8PairMinGroups = 1024;
// A one-row int8 workgroup whose row is at most two 16-byte loads per lane
// of kQ8NarrowWaves wavefronts has that many wavefronts instead of
// kGroupWaves: half the wavefronts, two loads per lane in flight (MI355X,
// µs, int8 with fp16 x, workgroups of 4 / 2 / 1 wavefronts: 4096 × 4096
// 4.76 / 4.69 / 4.87, 2048 × 4096 3.41 / 3.39 / 3.52; bf16 x 4096 × 4096
// 4.86 / 4.75 / 4.86; two rows per workgroup of 2 or 1 wavefronts 4.81,
// 5.15).
constexpr int kQ8NarrowWaves = 2;
// Threads per workgroup of the rows/wave and batched families.
constexpr int kBlock = 256;
// Below this many workgroups the rows-per-wave family stops giving each
// wavefront several row tiles, so that small problems still spread out.
// At most kRowsMaxTiles tiles, and with a full 32-lane row group two tiles
// while that still leaves kManyGroups workgroups: more, smaller workgroups
// stream tall matrices faster (MI355X, 2^20 rows, µs with 8 -> 4 -> 2
// tiles: fp32 K = 16 11.96, 11.96, 12.31; K = 32 21.71, 21.52, 22.17;
// K = 64 40.89, 40.19, 40.00; K = 128 80.59, 78.05, 76.94; bf16 K = 256
// 80.18, 77.77, 76.65; fp32 2^22 × 16 46.04, 44.31, 44.32; but fp32
// 2^18 × 128 20.44, 20.31, 21.29).
constexpr int64_t kTargetGroups = 1024;
constexpr int64_t kWaveMaxGroups = 16384;
constexpr int kRowsMaxTiles = 4;
constexpr int kRowsMinSplitLanes = 8;
constexpr int kRowsMaxBatch = 6;
constexpr int64_t kManyGroups = 65536;

struct Plan {
    int family = -1;
    int vector_loads = 0;
    int chunk_elems = 1;
    int lanes_per_row = 0;
    int rows_per_wave = 0;
    int row_tiles = 0;
    int waves_per_group = 0;
    int rows_per_group = 0;
    int batch = 0;
    int passes = 0;
    int block = 0;
    int lds_bytes = 0;
    int splits = 1;       // K-slices per row (split-K), else 1
    int slice_elems = 0;  // elements per slice (split-K), else K
    int x_in_registers = 0;  // workgroup per row: x kept in registers across its rows
    int rounding_chain = 0;  // bound on the fp32 roundings between a product and its output
    int column_blocks = 1;   // batched: launches (passes over A), each for a block of vectors
    int64_t grid = 0;     // workgroups (split-K: rows × slices)
};

inline int element_bytes(int dtype) { return dtype == F32 ? 4 : (dtype == Q8 ? 1 : 2); }

inline int next_pow2(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Loads per lane per batch for a row that gives each lane `per_lane` loads:
// as few batches of at most `cap` as possible, all of one size, so that no
// batch carries more clamped, discarded loads than rounding needs (a batch
// larger than the row costs registers and clamped loads: bf16 8192 × 1024
// with a wavefront per row, µs, batches of 8 / 2: 7.31 / 4.37).
inline int fitted_batch(int64_t per_lane, int cap) {
    if (per_lane < 1) return 1;
    return (int)ceil_div(per_lane, ceil_div(per_lane, (int64_t)cap));
}

// Argument checks shared by every entry point (see the header's "Errors").
inline int validate(int dtype, int M, int K, int lda, int nvec, uintptr_t A,
                    uintptr_t X, uintptr_t bias, uintptr_t Y) {
    if (dtype < F32 || dtype > BF16) return INVALID;
    if (M < 0 || K < 0 || lda < K) return INVALID;
    if (nvec < 1 || nvec > kMaxVectors) return INVALID;
    const uintptr_t s = (uintptr_t)element_bytes(dtype);
    if (M > 0 && K > 0 && (A == 0 || X == 0)) return INVALID;
    if (M > 0 && Y == 0) return INVALID;
    if (A % s != 0 || X % s != 0 || bias % 4 != 0 || Y % 4 != 0) return INVALID;
    return OK;
}

// Argument checks of the int8-weight entry points: Q int8 with row pitch
// ldq >= K, x in float type xdtype, one fp32 scale per row.
inline int validate_q8(int xdtype, int M, int K, int ldq, uintptr_t Q, uintptr_t scale,
                       uintptr_t x, uintptr_t bias, uintptr_t y) {
    if (xdtype < F32 || xdtype > BF16) return INVALID;
    if (M < 0 || K < 0 || ldq < K) return INVALID;
    if (M > 0 && K > 0 && (Q == 0 || x == 0)) return INVALID;
    if (M > 0 && (y == 0 || scale == 0)) return INVALID;
    if (x % (uintptr_t)element_bytes(xdtype) != 0 || scale % 4 != 0 || bias % 4 != 0 ||
        y % 4 != 0)
        return INVALID;
    return OK;
}

// 16-byte loads of int8 rows: Q and x 16-byte aligned; the row pitch may
// leave rows unaligned, as for one vector of the other types.
inline bool vector_ok_q8(int ldq, uintptr_t Q, uintptr_t x) {
    (void)ldq;
    return Q % kLoadBytes == 0 && x % kLoadBytes == 0;
}

// 16-byte loads need 16-byte aligned A and x (or X).  The row pitch and K
// may leave rows and X columns unaligned: the chunk loads take
// element-aligned addresses, and one unaligned 16-byte load beats eight
// element loads (MI355X, bf16 4096 × 4100 9.64 -> 6.98 µs, 384 × 43690
// 12.88 -> 8.97, 6144 × 2730 9.14 -> 7.01; fp32 4096 × 4097 13.97 -> 12.06;
// only where few rows leave CUs idle is it no faster: bf16 192 × 87381
// 12.25 -> 12.63).
inline bool vector_ok(int dtype, int K, int lda, int nvec, uintptr_t A, uintptr_t X) {
    (void)dtype, (void)K, (void)lda, (void)nvec;
    return A % kLoadBytes == 0 && X % kLoadBytes == 0;
}

// The matrix-core batched kernel reads whole aligned 16-byte operand rows:
// A and X aligned, and the row pitch and K whole 16-byte units.
inline bool mfma_rows_ok(int dtype, int K, int lda, uintptr_t A, uintptr_t X) {
    const int64_t s = element_bytes(dtype);
    return A % kLoadBytes == 0 && X % kLoadBytes == 0 && ((int64_t)lda * s) % kLoadBytes == 0 &&
           ((int64_t)K * s) % kLoadBytes == 0;
}

// Plan for a problem whose 16-byte-load eligibility `vec` the caller has
// decided (one matrix: vector_ok(); several: all of them).
// Row tiles per wavefront for several row-stacked matrices: every tile's row
// looks up its matrix per lane, which costs registers.
constexpr int kMultiMaxRowTiles = 2;

// rows per workgroup of an int8 plan of the workgroup-per-row family
inline int q8_group_rows(int64_t M, int64_t K, int x_bytes, bool vec) {
    if (!vec || ceil_div(M, (int64_t)2) < kQ8PairMinGroups) return 1;
    return (M > kQ8OneRowMaxRows || K * x_bytes >= kQ8PairMinXBytes) ? 2 : 1;
}

// Whether a single-vector problem keeps x in registers (see
// kGroupStreamMinXBytes) with at least two rows per workgroup.
inline bool stream_fits(int dtype, int64_t M, int64_t K, bool vec, int max_group_rows) {
    if (dtype == Q8 || !vec || max_group_rows < 2) return false;
    const int64_t elems = kLoadBytes / element_bytes(dtype);
    if (K % elems != 0 || K * element_bytes(dtype) <= kGroupStreamMinXBytes) return false;
    const int64_t chunks = ceil_div(K / elems, (int64_t)kWave * kGroupStreamWaves);
    return chunks <= kGroupStreamMaxChunks && ceil_div(M, 2) >= kGroupTileMinGroups;
}

// `vec`: 16-byte loads of A and x (or X) are possible; `mfma_rows`: with
// several vectors, also every row and X column starts 16-byte aligned (the
// matrix-core kernel reads aligned operand rows); `q8_x_bytes`: for int8
// weights, the bytes of one x element.
inline int make_plan_vec(int dtype, int M, int K, int nvec, bool vec, int family, Plan* out,
                         int max_row_tiles = 8, int max_group_rows = kGroupStreamRows,
                         int max_wave_tiles = kWaveBatch, int max_group_waves = kGroupWideWaves,
                         bool mfma_rows = false, int q8_x_bytes = 2) {
    if (dtype < F32 || dtype > Q8 || M < 0 || K < 0 || nvec < 1 || nvec > kMaxVectors)
        return INVALID;

    Plan p;
    const int nvec_all = nvec;
    p.vector_loads = vec ? 1 : 0;
    p.chunk_elems = p.vector_loads ? kLoadBytes / element_bytes(dtype) : 1;
    // loads needed to cover one row (the last may be a partial, element-wise tail)
    const int64_t loads = ceil_div(K, p.chunk_elems);
    const int64_t full = K / p.chunk_elems;

    // the matrix-core kernel reads every 8-element group of a row with one
    // aligned 16-byte load
    const bool mfma_ok = dtype != F32 && p.vector_loads && mfma_rows && K % 8 == 0;

    int fam = family;
    const bool long_or_many = loads >= kGroupLongRowLoads ||
                              (M >= kGroupManyRows && loads >= kGroupManyRowsMinLoads);
    if (fam == AUTO) {
        if (nvec > 1)
            fam = mfma_ok ? BATCHED_MFMA : BATCHED;
        else if (loads <= kRowsPerWaveMaxLanes)
            fam = ROWS_PER_WAVE;
        else if (M <= kGroupMaxRows || long_or_many ||
                 (M <= kGroupMidRows && loads >= kGroupMidMinLoads) ||
                 (dtype == Q8 && M <= kQ8GroupMaxRows && loads >= kGroupMidMinLoads) ||
                 stream_fits(dtype, M, K, p.vector_loads != 0, max_group_rows))
            fam = GROUP_PER_ROW;
        else
            fam = WAVE_PER_ROW;
    }
    const bool batched = fam == BATCHED || fam == BATCHED_MFMA;
    if (!batched && nvec != 1) return INVALID;
    // int8 weights run the three single-vector row families only
    if (dtype == Q8 && fam != ROWS_PER_WAVE && fam != WAVE_PER_ROW && fam != GROUP_PER_ROW)
        return INVALID;
    if (batched && dtype == F32) return INVALID;
    if (fam == BATCHED_MFMA && !mfma_ok) return INVALID;

    p.family = fam;
    switch (fam) {
    case ROWS_PER_WAVE: {
        if (loads > kRowsPerWaveMaxLanes) return INVALID;
        p.lanes_per_row = next_pow2(loads < 1 ? 1 : loads);
        p.rows_per_wave = kWave / p.lanes_per_row;
        p.waves_per_group = kBlock / kWave;
        p.batch = 1;
        // as many row tiles per wavefront as keeps >= kTargetGroups groups
        p.row_tiles = 1;
        // a load count that is not a power of two leaves lanes of a
        // power-of-two row group idle: for very tall single matrices, fewer
        // lanes per row (at least 8) with several loads each, when that
        // wastes fewer loads.  MI355X, 2^20 rows, µs: fp32 K = 72 58.6 ->
        // 53.0, K = 80 60.7 -> 52.2, K = 96 66.2 -> 57.1; bf16 K = 160 62.3 ->
        // 52.2, 192 68.0 -> 57.2; fp16 K = 176 63.3 -> 59.9.  But fp32 2^18 ×
        // 80 13.15 -> 14.45 (the row tiles of the power-of-two group won
        // there), and 4 lanes per row lost everywhere but K = 80/160 (fp32
        // 2^20 × 40 25.7 -> 37.6).
        // (int8 rows keep one load per lane: their rows kernels exist for
        // batches of one only below 64 lanes per row)
        if (dtype != Q8 && p.vector_loads && max_wave_tiles > 1 && loads > 2 &&
            p.lanes_per_row != loads) {
            int best_l = p.lanes_per_row, best_b = 1;
            int64_t best_waste = p.lanes_per_row - loads;
            for (int l = p.lanes_per_row / 2; l >= kRowsMinSplitLanes; l /= 2) {
                const int64_t b = ceil_div(loads, (int64_t)l);
                if (b > kRowsMaxBatch) break;
                const int64_t grid = ceil_div(M, (int64_t)(kWave / l) * p.waves_per_group);
                if (grid >= kWaveMaxGroups && l * b - loads < best_waste) {
                    best_waste = l * b - loads;
                    best_l = l;
                    best_b = (int)b;
                }
            }
            if (best_b > 1) {
                p.lanes_per_row = best_l;
                p.rows_per_wave = kWave / best_l;
                p.batch = best_b;
                break;  // one row tile
            }
        }
        if (p.vector_loads) {
            const int cap = max_row_tiles < kRowsMaxTiles ? max_row_tiles : kRowsMaxTiles;
            auto groups = [&](int u) {
                return ceil_div(M, (int64_t)u * p.rows_per_wave * p.waves_per_group);
            };
            for (int u = cap; u > 1; u >>= 1) {
                if (groups(u) >= kTargetGroups) {
                    p.row_tiles = u;
                    break;
                }
            }
            if (p.lanes_per_row == kRowsPerWaveMaxLanes && p.row_tiles > 2 && groups(2) >= kManyGroups)
                p.row_tiles = 2;
        }
        break;
    }
    case WAVE_PER_ROW: {
        p.lanes_per_row = kWave;
        p.rows_per_wave = 1;
        p.waves_per_group = kBlock / kWave;
        // (bf16 8192 × 2048, µs, batches of 8 / 4: 8.38 / 6.62)
        const int64_t per_lane = ceil_div(full, (int64_t)kWave);
        p.batch = fitted_batch(per_lane, kWaveBatch);
        p.row_tiles = 1;
        if (dtype != Q8 && p.vector_loads) {
            // very many short rows: a wavefront takes several rows (one row
            // tile each, all their loads in flight, at most kWaveBatch per
            // lane) until at most kWaveMaxGroups workgroups remain; launching
            // a workgroup costs about 0.2 ns (an empty kernel of 16384
            // workgroups takes 4.5 µs), so 2^20 rows at one per wavefront
            // were bound by the launch (fp32 2^20 × 256: 200 µs)
            for (int u = 1; u <= max_wave_tiles && u * p.batch <= kWaveBatch; u *= 2) {
                p.row_tiles = u;
                if (ceil_div(M, (int64_t)u * p.waves_per_group) <= kWaveMaxGroups) break;
            }
        }
        if (dtype == Q8) {
            // int8 rows: x chunks are 2-4 times the weight chunk, so batches
            // stop at kQ8Batch and two rows share every x chunk when there
            // are rows enough
            p.batch = fitted_batch(per_lane, kQ8Batch);
            if (ceil_div(M, 2 * (kBlock / kWave)) >= kQ8PairRowsMinGroups) p.row_tiles = 2;
        }
        break;
    }
    case GROUP_PER_ROW: {
        p.lanes_per_row = kWave * kGroupWaves;
        p.rows_per_wave = 0;  // a row spans the whole workgroup
        p.waves_per_group = kGroupWaves;
        // batches of at most 8 loads per lane (int8: 4), fitted to the row
        // (bf16 4096 × 14336: 7.  18.17 µs with batches of 8, 17.94 with 7)
        const int64_t per_lane = ceil_div(full, (int64_t)p.lanes_per_row);
        p.batch = fitted_batch(per_lane, dtype == Q8 ? kQ8Batch : kGroupBatch);
        // rows per workgroup (one x chunk serves all of them)
        int u = 1;
        const int umax = max_group_rows;
        const int64_t xbytes = (int64_t)K * element_bytes(dtype);
        if (dtype == Q8) {
            u = q8_group_rows(M, K, q8_x_bytes, p.vector_loads != 0);
            if (u == 1 && p.vector_loads && full <= 2 * kWave * kQ8NarrowWaves) {
                p.waves_per_group = kQ8NarrowWaves;
                p.lanes_per_row = kWave * kQ8NarrowWaves;
                p.batch = fitted_batch(ceil_div(full, (int64_t)p.lanes_per_row), kQ8Batch);
            }
        }
        // x in registers across 2-4 rows for an x of more than 8 KiB that
        // fits 6 chunks per lane (int8 weights: 4, or 3 with fp32 x, their x
        // chunks taking 8 or 16 registers each; more spilled).  int8 weights read 2 or 4 x bytes
        // per weight byte, so fetching x once per 4 rows pays off there too
        // (µs, workgroup of 2 rows / x in registers over 4: fp16 x 4096 ×
        // 11008 9.66 / 9.33, 4096 × 14336 11.81 / 11.01, 1024 × 16384 5.96 /
        // 4.84; bf16 x 4096 × 11008 9.70 / 9.20; fp32 x 4096 × 4096 5.49 /
        // 5.24, 4096 × 8192 9.67 / 8.14).
        const int64_t stream_x_bytes = dtype == Q8 ? (int64_t)K * q8_x_bytes : xbytes;
        const int max_chunks = dtype != Q8 ? kGroupStreamMaxChunks
                                           : (q8_x_bytes == 4 ? kQ8StreamMaxChunksWideX : kQ8StreamMaxChunks);
        if (stream_x_bytes > kGroupStreamMinXBytes) {
            const int64_t lanes = (int64_t)kWave * kGroupStreamWaves;
            const int64_t chunks = ceil_div(full, lanes);
            if (p.vector_loads && full * p.chunk_elems == K && chunks <= max_chunks) {
                int r = kGroupStreamRows < umax ? kGroupStreamRows : umax;
                while (r > 1 && ceil_div(M, r) < kGroupTileMinGroups) r /= 2;
                if (r > 1) {
                    p.x_in_registers = 1;
                    p.waves_per_group = kGroupStreamWaves;
                    p.lanes_per_row = (int)lanes;
                    p.batch = (int)chunks;  // every chunk of a row in flight
                    u = r;
                }
            }
        }
        if (dtype != Q8 && !p.x_in_registers && xbytes > kGroupShareMinXBytes) {
            const int ushare = umax < kGroupMaxTileRows ? umax : kGroupMaxTileRows;
            while (2 * u <= ushare && 2 * u * p.batch <= kGroupTileLoads &&
                   ceil_div(M, 2 * u) >= kGroupTileMinGroups)
                u *= 2;
        }
        p.row_tiles = u;
        const int wide = u == 1 ? kGroupWideWaves : kGroupWidePairWaves;
        if (!p.x_in_registers && dtype != Q8 && wide <= max_group_waves && M < kGroupWideMaxRows &&
            per_lane > p.batch) {
            p.waves_per_group = wide;
            p.lanes_per_row = kWave * wide;
            p.batch = fitted_batch(ceil_div(full, (int64_t)p.lanes_per_row), kGroupBatch);
        }
        p.lds_bytes = (int)(p.waves_per_group * u * sizeof(float));
        break;
    }
    case BATCHED:
        // more than kValuVectors vectors run as column blocks of at most
        // kValuVectors (one launch and one pass over A each); the plan is
        // the first block's
        if (nvec > kValuVectors) nvec = kValuVectors;
        p.rows_per_wave = batched_rows(M, nvec);
        // (the K-split forms take one row per group of wavefronts)
        p.lanes_per_row = kWave * (p.rows_per_wave == 1 ? batched_split(M, nvec) : 1);
        p.waves_per_group = kBlock / kWave;
        p.batch = batched_batch(nvec);
        p.row_tiles = 1;
        break;
    case GATED_SILU: {
        // a workgroup per row pair: 4 wavefronts for long rows or tall
        // matrices, else one wavefront (no LDS, no barrier)
        const int w = (M <= kGroupMaxRows || long_or_many) ? kGroupWaves : 1;
        p.lanes_per_row = kWave * w;
        p.rows_per_wave = 0;
        p.waves_per_group = w;
        const int64_t per_lane = ceil_div(full, (int64_t)p.lanes_per_row);
        p.batch = fitted_batch(per_lane, kGroupBatch);
        p.row_tiles = 1;
        p.lds_bytes = (int)(w * 2 * sizeof(float));
        break;
    }
    case BATCHED_MFMA:
        // each wavefront: 4 lanes per row and step, 16 rows; rows span the group
        p.row_tiles = mfma_row_groups(M, nvec);
        p.rows_per_wave = mfma_group_rows(M, nvec) * p.row_tiles;
        p.waves_per_group = mfma_waves(M, p.rows_per_wave);
        p.lanes_per_row = 4 * p.waves_per_group;
        p.batch = mfma_chunk(nvec, p.row_tiles);
        p.lds_bytes = mfma_lds_bytes(nvec, p.waves_per_group, p.row_tiles);
        break;
    default:
        return INVALID;
    }
    p.block = p.waves_per_group * kWave;
    if (fam == GROUP_PER_ROW)
        p.rows_per_group = p.row_tiles;
    else if (fam == GATED_SILU)
        p.rows_per_group = 1;
    else if (fam == BATCHED_MFMA)
        p.rows_per_group = p.rows_per_wave;
    else if (fam == BATCHED)  // lanes_per_row / 64 wavefronts share each row
        p.rows_per_group = p.rows_per_wave * (p.waves_per_group * kWave / p.lanes_per_row);
    else
        p.rows_per_group = p.rows_per_wave * p.row_tiles * p.waves_per_group;
    p.grid = ceil_div(M, p.rows_per_group);
    p.slice_elems = K;
    if (fam == BATCHED_MFMA)  // 64-wide steps (the last may be partial) per wavefront
        p.passes = mfma_step_range(K, p.waves_per_group, 0).end;
    else
        p.passes = (int)ceil_div(full, (int64_t)p.lanes_per_row);
    if (p.grid > 0x7fffffff) return INVALID;

    // The rounding-chain bound (+ 1: the bias, or the int8 scale and bias in
    // one fused multiply-add, added last).  The matrix-core kernel's 4-tile
    // form accumulates in place, so for long rows its vectors run as blocks
    // of 32 (2 tiles, compensated; one pass over A per block).
    int64_t chain = 0;
    switch (fam) {
    case BATCHED_MFMA: {
        int blk = nvec;
        chain = mfma_chain(K, p.waves_per_group, mfma_chunk(blk, p.row_tiles), mfma_tiles(blk) <= 2) + 1;
        if (chain > kMaxRoundingChain && mfma_tiles(nvec) > 2) {
            blk = 32;
            p.column_blocks = (int)ceil_div(nvec, (int64_t)blk);
            p.batch = mfma_chunk(blk);
            p.lds_bytes = mfma_lds_bytes(blk, p.waves_per_group);
            chain = mfma_chain(K, p.waves_per_group, mfma_chunk(blk), true) + 1;
        }
        break;
    }
    case BATCHED:
        // one accumulator per (row, vector) per run of batches, FMA per element
        p.column_blocks = (int)ceil_div(nvec_all, (int64_t)kValuVectors);
        chain = batched_chain(K, p.chunk_elems, p.batch, batched_run(nvec, p.batch, p.chunk_elems),
                              p.lanes_per_row / kWave) +
                1;
        break;
    default:
        if (p.x_in_registers)  // one batch per row, no running sum
            chain = (p.batch + 1) / 2 * p.chunk_elems + 1 + ceil_log2(kWave) + (p.waves_per_group - 1) + 1;
        else  // (only the workgroup families fold several wavefronts' partials)
            chain = valu_chain(K, p.chunk_elems, p.lanes_per_row,
                               p.lanes_per_row < kWave ? p.lanes_per_row : kWave, p.batch,
                               fam == GROUP_PER_ROW || fam == GATED_SILU ? p.waves_per_group : 1) +
                    1;
        break;
    }
    if (chain > kMaxRoundingChain) return INVALID;
    p.rounding_chain = (int)chain;
    *out = p;
    return OK;
}

// Slices for split-K.  `requested` = 0 chooses: 1 unless the rows are few
// and long (above), else as many slices as keep M × splits within
// kTargetGroups workgroups, each at least kSplitMinSliceLoads loads long.  `requested` >= 1 asks for that many (used as
// given, after rounding the slice up to whole 16-byte loads and capping at
// kSplitMaxSplits).  The slice is a whole number of 16-byte loads of every
// dtype, so 16-byte alignment of A and x carries over to every slice.
inline int split_geometry(int dtype, int M, int K, int requested, int* splits, int* slice) {
    if (dtype < F32 || dtype > BF16 || M < 0 || K < 0 || requested < 0) return INVALID;
    const int64_t granule = kLoadBytes / element_bytes(dtype);  // elements per load
    const int64_t loads = ceil_div(K, granule);
    int64_t want = requested;
    if (requested == 0) {
        want = 1;
        if (M > 0 && M < kSplitMaxRows && loads >= kSplitMinRowLoads) {
            // below 8 rows x is not shared between rows, so each workgroup
            // streams as many x bytes as A bytes: half as many workgroups
            const int64_t by_rows = (M < 8 ? kTargetGroups / 2 : kTargetGroups) / M;
            const int64_t by_len = loads / kSplitMinSliceLoads;
            want = by_rows < by_len ? by_rows : by_len;
            if (want >= 8) want -= want % 8;  // whole rounds of the 8 XCDs
            if (want < 2) want = 1;
        }
    }
    if (want > kSplitMaxSplits) want = kSplitMaxSplits;
    if (want < 1 || loads <= 1) want = 1;
    int64_t slice_loads = 1, n = 1;
    for (;;) {
        slice_loads = ceil_div(loads, want);
        if (requested == 0 && want > 1)  // whole wavefront-wide loads
            slice_loads = ceil_div(slice_loads, (int64_t)kWave) * kWave;
        if (slice_loads < 1) slice_loads = 1;
        n = ceil_div(loads, slice_loads);
        if (n < 1) n = 1;
        // an automatic count of 8 or more stays a multiple of 8 (rounding
        // the slice up can leave fewer slices than asked for)
        if (requested != 0 || n < 8 || n % 8 == 0 || want <= 8) break;
        want -= 8;
    }
    *splits = (int)n;
    *slice = n == 1 ? K : (int)(slice_loads * granule);
    return OK;
}

// Workspace bytes split-K needs: one fp32 partial per row and slice (none
// when one slice is chosen, which runs the single-pass families).
inline int64_t split_workspace_bytes(int M, int splits) {
    return splits > 1 ? (int64_t)M * splits * (int64_t)sizeof(float) : 0;
}

// Plan of a split-K call: pass 1 of family SPLIT_K (a workgroup of 4
// wavefronts per row and slice, grid = M × splits), or, with one slice, the
// automatic single-pass plan.
inline int make_split_plan(int dtype, int M, int K, bool vec, int requested, Plan* out) {
    int splits = 1, slice = K;
    if (split_geometry(dtype, M, K, requested, &splits, &slice) != OK) return INVALID;
    if (splits == 1) {
        if (make_plan_vec(dtype, M, K, 1, vec, AUTO, out) != OK) return INVALID;
        out->splits = 1;
        out->slice_elems = K;
        return OK;
    }
    Plan p;
    p.family = SPLIT_K;
    p.vector_loads = vec ? 1 : 0;
    p.chunk_elems = p.vector_loads ? kLoadBytes / element_bytes(dtype) : 1;
    const int64_t full = slice / p.chunk_elems;  // whole chunks of a full slice
    p.lanes_per_row = kWave * kGroupWaves;
    p.rows_per_wave = 0;
    p.waves_per_group = kGroupWaves;
    const int64_t per_lane = ceil_div(full, (int64_t)p.lanes_per_row);
    p.rows_per_group = M >= 2 ? kSplitRowsPerGroup : 1;
    p.batch = fitted_batch(per_lane, kGroupBatch);
    p.row_tiles = 1;
    p.block = p.waves_per_group * kWave;
    p.lds_bytes = (int)(kGroupWaves * p.rows_per_group * sizeof(float));
    p.splits = splits;
    p.slice_elems = slice;
    // one workgroup per (row tile, slice)
    p.grid = ceil_div((int64_t)M, (int64_t)p.rows_per_group) * splits;
    if (p.grid * p.block > 0xffffffffLL) return INVALID;  // HIP's 32-bit grid size
    p.passes = (int)per_lane;
    // pass 1 over a slice (no bias), then the reduce: each lane adds up to
    // ceil(splits/64) partials in turn, a 64-lane tree, the bias
    const int64_t chain = valu_chain(slice, p.chunk_elems, p.lanes_per_row, kWave, p.batch,
                                     p.waves_per_group) +
                          ceil_div(splits, (int64_t)kWave) + ceil_log2(kWave) + 1;
    if (chain > kMaxRoundingChain) return INVALID;
    p.rounding_chain = (int)chain;
    *out = p;
    return OK;
}

// Workgroups of a single matrix's wave-per-row plan (one row per wavefront,
// one row tile, 16-byte loads): kBlock / kWave wavefronts, or
// kNarrowRowsWaves when that spreads the grid more evenly over the kCUs
// compute units, i.e. when the busiest unit's share of workgroups, over the
// mean, is smaller (g workgroups: ceil(g / kCUs)·kCUs / g).  A grid of 384
// four-wavefront workgroups leaves half the units two and half one; 768 of
// two leave every unit three.  MI355X, bf16 K = 4096, µs, 4 / 2 wavefronts:
// 1280 rows 3.97 / 3.85, 1536 4.09 / 3.93, 2304 5.13 / 4.89, 2560 5.23 /
// 5.09, 3584 6.36 / 6.24, 5632 8.58 / 8.56; fp32 1536 × 2048 4.06 / 3.79;
// where the shares tie, 4 stays (768 3.04 / 3.26, 1024 3.22 / 3.45, 1792
// 4.22 / 4.36, 2048 4.32 / 4.44, 2816 5.38 / 5.58, 4096 6.66 / 6.73).
constexpr int kNarrowRowsWaves = 2;
inline bool narrow_rows_balance_better(int64_t M) {
    const int64_t g4 = ceil_div(M, (int64_t)(kBlock / kWave)), g2 = ceil_div(M, (int64_t)kNarrowRowsWaves);
    // ceil(g2/C)·C/g2 < ceil(g4/C)·C/g4, cross-multiplied
    return g4 > 0 && ceil_div(g2, kCUs) * g4 < ceil_div(g4, kCUs) * g2;
}
inline void balance_rows_workgroups(int dtype, int nvec, int64_t M, Plan* p) {
    if (p->family != WAVE_PER_ROW || dtype == Q8 || nvec != 1 || p->row_tiles != 1 ||
        !p->vector_loads || !narrow_rows_balance_better(M))
        return;
    p->waves_per_group = kNarrowRowsWaves;
    p->block = kNarrowRowsWaves * kWave;
    p->rows_per_group = kNarrowRowsWaves;
    p->grid = ceil_div(M, (int64_t)p->rows_per_group);
}

inline int make_plan(int dtype, int M, int K, int lda, int nvec, uintptr_t A, uintptr_t X,
                     int family, Plan* out) {
    if (lda < K) return INVALID;
    const int rc = make_plan_vec(dtype, M, K, nvec, vector_ok(dtype, K, lda, nvec, A, X), family,
                                 out, 8, kGroupStreamRows, kWaveBatch, kGroupWideWaves,
                                 mfma_rows_ok(dtype, K, lda, A, X));
    if (rc == OK) balance_rows_workgroups(dtype, nvec, M, out);
    return rc;
}

}  // namespace gemvplan
