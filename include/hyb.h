/*
 * hyb.h -- C ABI of libhyb: tile-hybrid dense / 2:4 sparse weights for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  A weight matrix W (n x k, out x in, row-major) is cut
 * into b1 x b2 tiles; each tile is either dense or 2:4 sparse, chosen per tile
 * by a caller-supplied map (PATCH: Learnable Tile-level Hybrid Sparsity for
 * LLMs, gist.science, section 2 "Meccanismo Principale").  In a sparse tile
 * every row keeps, in each aligned group of four columns, two entries -- one
 * of the six two-of-four patterns (same page, section 2 "Distribuzioni
 * Apprendibili") -- and the matrix is stored compressed: two values per group
 * plus a 4-bit code, a constant number of slots per group (SparseDecoding,
 * ai.info, authors' abstract: bitmask-indexed N:M storage read with a fixed
 * stride).  The products y = W' x (decode, 1..16 tokens) and Y = X W'^T
 * (prefill) read that compressed form; W' is W with the dropped entries set
 * to zero, so results equal the plain product with W'.
 *
 * Which two entries are kept: the two largest |w| of the group, |w| compared
 * as the integer (bits & 0x7FFF), equal magnitudes going to the lower column
 * (magnitude projection: 3BASiL, gist.science, section 2 "Aggiornamenti
 * Chiusi"; the pages learn this choice instead, which needs training data).
 *
 * Stream format "HYB1" (element indices count 16-bit words):
 *   tile t = tn*tiles_k + tk; dense tiles take dense slots 0,1,.. and sparse
 *   tiles sparse slots 0,1,.. in increasing t; tidx[t] = slot for a dense
 *   tile and ~slot for a sparse one.
 *   dense  slot s, element (r, c):
 *       s*b1*b2 + (r/16)*16*b2 + (c/32)*512 + ((c%32)/8)*128 + (r%16)*8 + c%8
 *   values slot s, row r, group g (columns 4g..4g+3), kept j = 0, 1 (ascending
 *       column):  s*b1*b2/2 + (r/16)*8*b2 + (g/16)*512 + ((g%16)/4)*128
 *                 + (r%16)*8 + (g%4)*2 + j
 *   meta   16-bit little-endian words; the group's nibble is in word
 *       s*b1*b2/16 + (r/16)*b2 + (((g%16)/4)*16 + r%16)*(b2/64) + g/16
 *       at bits 4*(g%4)..4*(g%4)+3;  HYB_META_IDX2: i0 | i1<<2,
 *       HYB_META_MASK4: 1<<i0 | 1<<i1  (i0 < i1 the kept columns).
 *   4:8 tiles (HYB_META_MASK8).  PATCH section 5 "Significato" names 4:8
 *   as the next N:M pattern for the same scheme, and SparseDecoding's kernel
 *   reads N:M with bitmask indices.  Each aligned group of eight columns
 *   keeps its four largest |w| (same key and tie rule); a sparse tile has
 *   the same byte counts as a 2:4 one.
 *   values slot s, row r, group h (columns 8h..8h+7), kept j = 0..3
 *       (ascending column):  s*b1*b2/2 + (r/16)*8*b2 + (h/8)*512
 *                 + ((h%8)/2)*128 + (r%16)*8 + (h%2)*4 + j
 *   meta   the mask byte (bit p set = column 8h+p kept) sits in the word of
 *       the 2:4 group g = 2h above, at bits 8*(h%2)..8*(h%2)+7.
 *   Every 1 KiB of the dense or value stream is one 16-row slab piece that a
 *   64-lane wavefront loads with one 16-byte load per lane.
 *
 * Conventions.
 *   - All pointers to device memory are plain device addresses (from
 *     hipMalloc or any allocator on the same device); the library never
 *     allocates or frees device memory and keeps no mutable global state
 *     apart from a per-device cache of the compute-unit count (used to
 *     pick launch shapes).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device calls enqueue work and return; the caller synchronises.
 *   - Every argument is checked on the host before anything is enqueued; a
 *     failed check returns a non-zero status, enqueues nothing and leaves a
 *     message for hyb_last_error() (thread-local).
 *   - Outputs must not overlap inputs.
 *   - Entries of tidx that name a slot outside [0, n_dense) or
 *     [0, n_sparse) are not reported; the kernels skip such tiles (they add
 *     nothing and write nothing) so they never read outside the streams.
 *     Metadata nibbles outside the six valid codes (mask bytes without
 *     exactly four bits set) give unspecified values for that group (never
 *     an out-of-bounds access).
 */
#ifndef HYB_H_
#define HYB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hyb_status;
enum {
  HYB_OK = 0,
  HYB_ERR_INVALID_ARG = 1, /* null pointer, bad stride, bad alignment, bad value */
  HYB_ERR_SHAPE = 2,       /* n % b1 or k % b2 non-zero, negative sizes, m out of range */
  HYB_ERR_DTYPE = 3,       /* unknown element or output type */
  HYB_ERR_UNSUPPORTED = 4, /* tile size outside {64, 128, 256} */
  HYB_ERR_FORMAT = 5,      /* layout magic / version / sizes inconsistent */
  HYB_ERR_HIP = 6          /* a HIP launch or runtime call failed */
};

enum { HYB_F16 = 1, HYB_BF16 = 2, HYB_F32 = 3 };    /* element types */
enum { HYB_META_IDX2 = 1, HYB_META_MASK4 = 2,       /* metadata codes (2:4 tiles) */
       HYB_META_MASK8 = 3 };                         /* 4:8 tiles, see above */

#define HYB_MAGIC 0x31425948u /* "HYB1" little-endian */
#define HYB_VERSION 1u
#define HYB_ABI_VERSION 1
#define HYB_MAX_GROUP 16 /* matrices per hyb_gemv_grouped call */
#define HYB_MAX_RANK 256 /* largest rank of hyb_gemv_lowrank */

/* Plain-old-data description of one packed matrix; filled by hyb_plan and
 * also usable as a serialised header (all fields fixed-width). */
typedef struct {
  uint32_t magic, version; /* HYB_MAGIC, HYB_VERSION */
  int64_t n, k;            /* W is n x k (out_features x in_features) */
  int32_t b1, b2;          /* tile rows x tile columns */
  int32_t dtype, meta;     /* HYB_F16 | HYB_BF16; HYB_META_IDX2 | HYB_META_MASK4 | HYB_META_MASK8 */
  int64_t tiles_n, tiles_k, n_dense, n_sparse;
  int64_t dense_bytes, val_bytes, meta_bytes, tidx_bytes;
} hyb_layout;

/* Device addresses of the four streams of one packed matrix (owned by the
 * caller).  dense, val and meta must be 16-byte aligned; tidx 4-byte
 * aligned.  A stream of zero bytes may be NULL. */
typedef struct {
  void* dense;
  void* val;
  void* meta;
  int32_t* tidx;
} hyb_packed;

/* Plan a packed layout (host only, no device work; the tile-map step of
 * PATCH section 2 "Meccanismo Principale").
 *   n, k      matrix shape, n % b1 == 0 and k % b2 == 0 (0 allowed)
 *   b1, b2    tile shape; any positive b1 % 16 == 0, b2 % 64 == 0 is planned,
 *             the device calls accept b1, b2 in {64, 128, 256}
 *   tile_map  host uint8[tiles_n * tiles_k], row-major over the tile grid,
 *             0 = dense, 1 = 2:4 sparse; may be NULL when there are no tiles
 *   out       receives the layout (byte sizes of the four streams)
 *   tidx_out  host int32[tiles_n * tiles_k] receiving the tile index, or NULL
 * The caller allocates the streams and copies tidx_out to packed.tidx. */
hyb_status hyb_plan(int64_t n, int64_t k, int32_t b1, int32_t b2, int32_t dtype,
                    int32_t meta, const uint8_t* tile_map, hyb_layout* out,
                    int32_t* tidx_out);

/* Check a layout held by the caller (host only, nothing enqueued): the
 * magic and version, the geometry rules of hyb_plan, and that the tile
 * counts and stream sizes agree with each other -- e.g. a header read back
 * from a file.  Returns HYB_OK, HYB_ERR_INVALID_ARG (NULL), HYB_ERR_FORMAT
 * (magic, version, counts or sizes), HYB_ERR_SHAPE or HYB_ERR_DTYPE.  Tile
 * sizes outside {64, 128, 256} pass here; the device calls reject them. */
hyb_status hyb_layout_check(const hyb_layout* layout);

/* Pack W into the streams of `dst` (the pruning and compression of PATCH
 * section 2 with the magnitude rule above; SparseDecoding abstract for the
 * fixed-stride bitmask storage).
 *   w     device, n x k elements of layout->dtype, row stride ldw >= k
 *         elements, 16-byte aligned, ldw % 8 == 0
 *   dst   device streams sized as in *layout; dst->tidx must already hold
 *         the tile index from hyb_plan
 * Bit-exact: the streams depend only on the bits of W and the map. */
hyb_status hyb_pack(const hyb_layout* layout, const void* w, int64_t ldw,
                    const hyb_packed* dst, void* stream);

/* Rebuild W' (n x k, row stride ldw) from packed streams, the inverse of
 * hyb_pack: dense tiles as stored, sparse groups with their two values at
 * the coded columns and +0.0 at the other two (PATCH section 2 "Meccanismo
 * Principale": a sparse tile is the 2:4-pruned tile, the dropped entries
 * zero; SparseDecoding abstract for the bitmask-indexed storage read back).
 *   w_out  device, n x k elements of layout->dtype, row stride ldw >= k,
 *          16-byte aligned, ldw % 8 == 0 (ldw >= 0 even when n or k is 0)
 *   src    device streams as written by hyb_pack for *layout
 * Bit-exact: w_out depends only on the stream bytes. */
hyb_status hyb_unpack(const hyb_layout* layout, const hyb_packed* src, void* w_out,
                      int64_t ldw, void* stream);

/* Decode product, 0 <= m <= 16 tokens: Y[i, :] = W' X[i, :] for i < m
 * (SparseDecoding abstract: the decode-phase sparse matrix x vector product
 * over the compressed matrix).  Up to 4 tokens (16 on a matrix of at most
 * one 16-row slab per compute unit) the decode kernel runs; 5-16 tokens
 * otherwise run the matrix-core kernel, exactly as hyb_gemm routes them
 * (the decode kernel is bound by its vector arithmetic there).
 *   x       device, m x k of layout->dtype, row stride ldx >= k (elements),
 *           16-byte aligned, ldx % 8 == 0
 *   y       device, m x n, row stride ldy >= n, element type y_dtype in
 *           {HYB_F32, layout->dtype}; 16-bit outputs are rounded to nearest
 *           even from the fp32 sum
 * Products are exact in fp32 and summed in fp32; m == 0 returns HYB_OK with
 * nothing enqueued. */
hyb_status hyb_gemv(const hyb_layout* layout, const hyb_packed* w, const void* x,
                    int32_t m, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                    void* stream);

/* Grouped decode product: one launch (two when the matrices' sizes call
 * for different wavefront counts per slab, as hyb_gemv would pick for each
 * alone) multiplies the same x (0 <= m <= 16 tokens) by `count` packed
 * matrices, Y_g[i, :] = W'_g X[i, :]; a matrix that hyb_gemv would run on
 * the matrix cores (9-16 tokens on a long matrix) runs there in a launch of
 * its own, checked with the others before anything is enqueued.  A layer's
 * projections that read the same activations (q, k and v; gate and up) carry
 * their own tile maps and sparsities (PATCH, gist.science, section 3
 * "Contributi Chiave": attention stays denser, MLP matrices sparser), and the
 * smaller ones are too short to fill the GPU alone.
 *   count     0 <= count <= HYB_MAX_GROUP (0: no-op)
 *   layouts   host array of count layouts; every matrix must have the same k,
 *             b2, dtype and metadata kind (b1 and n may differ)
 *   w         host array of count stream descriptors
 *   x, m, ldx as for hyb_gemv (shared by all matrices)
 *   y         host array of count device pointers, matrix g's output m x n_g
 *   y_dtype   one output type for all (HYB_F32 or the weight dtype)
 *   ldy       host array of count row strides (ldy[g] >= n_g)
 * Every per-matrix check of hyb_gemv applies; outputs must not overlap each
 * other or the inputs.  Results are bitwise those of count hyb_gemv calls. */
hyb_status hyb_gemv_grouped(int32_t count, const hyb_layout* layouts, const hyb_packed* w,
                            const void* x, int32_t m, int64_t ldx, void* const* y,
                            int32_t y_dtype, const int64_t* ldy, void* stream);

/* Low-rank projection T = X V for a sparse + low-rank weight W ~ S + U V^T
 * (3BASiL, gist.science, section 1 "Il Problema": a sparse part plus a
 * rank-r part), U n x r and V k x r: the first of the two products of the
 * low-rank term X (U V^T)^T = (X V) U^T.  Any m >= 0.
 *   v      device, V stored transposed: rank rows of k values of `dtype`,
 *          row j (column j of V) at v + j * ldv; ldv >= k, ldv % 8 == 0,
 *          16-byte aligned
 *   rank   0 <= rank <= HYB_MAX_RANK (0: no-op)
 *   k      k >= 0, k % 8 == 0 (0: T is set to zero)
 *   dtype  HYB_BF16 or HYB_F16, the type of v and x
 *   x      device m x k, row stride ldx >= k, ldx % 8 == 0, 16-byte aligned
 *   t      device fp32 output m x rank, row stride ldt >= rank
 * Products are exact and summed in fp32 in a fixed order (the result is
 * deterministic).  0 <= m <= 16 * 65535 (one launch).  Decode sizes
 * (m <= 16) take one workgroup per row of V on the vector ALUs; larger m
 * runs on the matrix cores (exact products, fp32 sums), one workgroup per
 * 16 tokens. */
hyb_status hyb_lowrank_project(const void* v, int64_t ldv, int32_t rank, int64_t k, int32_t dtype,
                               const void* x, int32_t m, int64_t ldx, float* t, int64_t ldt,
                               void* stream);

/* Decode product of a sparse + low-rank weight, 0 <= m <= 16 tokens:
 * Y[i, :] = W' X[i, :] + U T[i, :], i.e. Y = X W'^T + T U^T, the second
 * product of X (S + U V^T)^T with S = W' packed here (3BASiL section 4
 * "Risultati Sperimentali" pairs 2:4 sparsity with rank 64).  T = X V
 * (m x rank) comes from hyb_lowrank_project; this call adds T U^T inside the
 * decode kernel, after each row's sparse sum (9-16 tokens that hyb_gemv
 * would run on the matrix cores run hyb_gemm_lowrank's kernel instead).
 *   layout, w, x, m, ldx, y, y_dtype, ldy  as for hyb_gemv
 *   t      device fp32, m x rank, row stride ldt >= rank, ldt % 4 == 0,
 *          16-byte aligned
 *   u      device, n x rank of layout->dtype, row stride ldu >= rank,
 *          ldu % 8 == 0, 16-byte aligned
 *   rank   0 <= rank <= HYB_MAX_RANK, rank % 8 == 0 (0: plain hyb_gemv)
 * The low-rank term is accumulated in fp32 (u widened, fp32 products), into
 * the same per-row sums as the sparse product. */
hyb_status hyb_gemv_lowrank(const hyb_layout* layout, const hyb_packed* w, const void* x,
                            int32_t m, int64_t ldx, const float* t, int64_t ldt, const void* u,
                            int64_t ldu, int32_t rank, void* y, int32_t y_dtype, int64_t ldy,
                            void* stream);

/* Sparse + low-rank product for any m >= 0: Y = X W'^T + T U^T as for
 * hyb_gemv_lowrank (3BASiL sections 1 and 4), with the same arguments and
 * checks.  The fused decode kernel runs where hyb_gemm would run the decode
 * kernel (m <= 4, or m <= 16 on short matrices); larger m the matrix-core
 * kernels, which add T U^T to each output tile before it is stored (fp32
 * products and sums, rank walked in order), so 16-bit outputs are rounded
 * once.  rank 0 is plain hyb_gemm. */
hyb_status hyb_gemm_lowrank(const hyb_layout* layout, const hyb_packed* w, const void* x,
                            int32_t m, int64_t ldx, const float* t, int64_t ldt, const void* u,
                            int64_t ldu, int32_t rank, void* y, int32_t y_dtype, int64_t ldy,
                            void* stream);

/* hyb_gemm_lowrank with a caller-held split-K workspace, as hyb_gemm_ws is
 * to hyb_gemm (for code under graph capture, where the library allocates
 * nothing, and callers that manage device memory).  The workspace size is
 * that of hyb_gemm_workspace_size for the same layout and m (the route does
 * not depend on the rank); workspace_bytes = 0 runs the same shape unsplit,
 * a positive size below the need -> HYB_ERR_INVALID_ARG.  Other arguments
 * and errors as hyb_gemm_lowrank. */
hyb_status hyb_gemm_lowrank_ws(const hyb_layout* layout, const hyb_packed* w, const void* x,
                               int32_t m, int64_t ldx, const float* t, int64_t ldt, const void* u,
                               int64_t ldu, int32_t rank, void* y, int32_t y_dtype, int64_t ldy,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Prefill product for any m >= 0 (PATCH section 2 "Inferenza e Deployment":
 * sparse tiles on the matrix units, dense tiles on dense kernels).  Same
 * arguments as hyb_gemv; m <= 4 runs the decode kernel (also m <= 16 when
 * the matrix has at most one 16-row slab per compute unit), larger m
 * the matrix-core kernels.  Where those split K over workgroups
 * (HYB_KERNEL_SPLIT of hyb_gemm_shape) they keep partial sums in a
 * workspace that the library allocates (hipMalloc, 64 MiB) at the first
 * such launch on a (device, stream) pair and holds until the process ends;
 * launches on one stream share it, so concurrent calls on different
 * streams stay safe.  Nothing is allocated on a stream that is being
 * captured into a graph: there (and if the allocation fails) the product
 * runs unsplit unless the stream already holds its workspace; hyb_gemm_ws
 * takes a caller-held one. */
hyb_status hyb_gemm(const hyb_layout* layout, const hyb_packed* w, const void* x,
                    int32_t m, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                    void* stream);

/* hyb_gemm with a caller-held workspace instead of the library's (for code
 * under graph capture, or callers that manage device memory themselves).
 * hyb_gemm_workspace_size gives the bytes the product needs on the current
 * device (0 when its route does not split K; m >= 0).  `workspace`: device
 * memory, 16-byte aligned, no initial contents needed, not read after the
 * call's work on `stream` completes; launches that overlap on one buffer
 * race.  workspace_bytes = 0 (workspace may be NULL) runs the same shape
 * unsplit; a positive size below the need -> HYB_ERR_INVALID_ARG.  Other
 * arguments and errors as hyb_gemm. */
hyb_status hyb_gemm_workspace_size(const hyb_layout* layout, int32_t m, size_t* bytes);
hyb_status hyb_gemm_ws(const hyb_layout* layout, const hyb_packed* w, const void* x,
                       int32_t m, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                       void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): hyb_gemm with no
 * allocation at all.  Where hyb_gemm would split K it uses a scratch array
 * that the library holds in static device memory, 64 MiB per GPU from the
 * library's load until the process ends, instead of a workspace (its
 * address is looked up once per device, at the first call there).  The
 * array keeps the last call's contents and needs no clearing; all calls on
 * one GPU share it, so calls that overlap on one GPU (concurrent streams or
 * host threads) race and must be serialised by the caller.  A product that
 * would need more than the array holds -> HYB_ERR_UNSUPPORTED (none does on
 * up to 256 CUs).  Arguments and other errors as hyb_gemm. */
hyb_status hyb_gemm_noalloc(const hyb_layout* layout, const hyb_packed* w, const void* x,
                            int32_t m, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                            void* stream);

/* Matrix-core kernel only, any m >= 0 (no switch to the decode kernel);
 * exposed so that the crossover can be measured.  Same arguments. */
hyb_status hyb_gemm_mfma(const hyb_layout* layout, const hyb_packed* w, const void* x,
                         int32_t m, int64_t ldx, void* y, int32_t y_dtype,
                         int64_t ldy, void* stream);

/* Diagnostics, host only (no device work, nothing enqueued): the kernel and
 * workgroup shape that hyb_gemm would launch for `m` >= 1 tokens on
 * `layout`'s matrix on the current device (its compute-unit count; 256, the
 * MI355X's, when no device is visible).  hyb_gemm_mfma launches the same for
 * m > 16, and for m <= 16 the register-fed shape of out[0] = 2 or 4.  Writes
 * out[4] = {kernel, token blocks of 16 per workgroup, wavefronts per
 * workgroup, 64-row groups per workgroup}: kernel HYB_KERNEL_DECODE (k_gemv;
 * out[1] = out[3] = 0, out[2] its wavefronts per 16-row slab),
 * HYB_KERNEL_REGISTER (k_gemm_rx, wavefronts splitting K), HYB_KERNEL_LDS
 * (k_gemm_lds, 4 row groups) or HYB_KERNEL_SPLIT (k_gemm_split with 1-2
 * row groups, the register-fed shape, or k_gemm_lds_split with 4 and 4 or
 * 8 token blocks, the LDS-fed 64- or 128-token shape: the (tile, K step)
 * units dealt out evenly over a fixed number of workgroups; or
 * k_gemm_lds_parts with 4 row groups and 12 or 16 token blocks, the 192- or
 * 256-token LDS tile with K cut into equal parts, one per workgroup; with
 * 16 token blocks and more tiles than CUs, a plain k_gemm_lds launch first
 * runs the leading 256-row blocks whose tiles fill whole rounds of the CUs,
 * and the parts cover the remaining blocks; partial tiles added by a second
 * kernel in a fixed order; it needs a workspace, which hyb_gemm holds per
 * device and stream).  Errors: as the layout checks of hyb_gemm; out NULL ->
 * HYB_ERR_INVALID_ARG; m < 1 -> HYB_ERR_SHAPE. */
enum { HYB_KERNEL_DECODE = 1, HYB_KERNEL_REGISTER = 2, HYB_KERNEL_LDS = 3, HYB_KERNEL_SPLIT = 4 };
hyb_status hyb_gemm_shape(const hyb_layout* layout, int32_t m, int32_t* out);

/* Measurement aid (no part of the product computation): reads `bytes`
 * bytes at `p` (device, 16-byte aligned) with the same non-temporal 16-byte
 * buffer loads the decode kernel uses, `grid` workgroups of 256 threads, and
 * writes one word per thread to `sink` (device, grid * 256 uint32).  It
 * gives the practical HBM read rate of this device for a given size, the
 * reference the decode kernel's rate is compared with (the spec peak is the
 * other).  bytes in [0, 2^31), grid in [1, 65535]. */
hyb_status hyb_stream_read(const void* p, int64_t bytes, uint32_t* sink, int32_t grid, void* stream);

const char* hyb_status_str(hyb_status s); /* static string, never NULL */
const char* hyb_last_error(void);         /* thread-local detail, "" if none */
int32_t hyb_abi_version(void);            /* HYB_ABI_VERSION */

#ifdef __cplusplus
}
#endif
#endif /* HYB_H_ */
