/*
 * mpb.h -- C ABI of libmpb, the MI355X (gfx950) mixed-precision MoE layer.
 *
 * The layer is the one PagedWeight runs inside its serving loop ("PagedWeight:
 * Efficient MoE LLM Serving with Dynamic Quality-Aware Weight Quantization",
 * §3.3 "Fused Mixed-Precision MoE Kernel"): top-K routing, expert gate_up with
 * SwiGLU, the down projection and the routing-weighted output accumulation,
 * with every expert weight read straight from Any-Precision bit-planes and
 * per-row lookup tables at the bitwidth q_i committed for its linear-block
 * (§3.1 "Paged Weight Representation").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Return value: 0 on success, a negative MPB_E_* code on failure. No C++
 *   exception crosses the ABI. mpb_last_error() gives a message for the last
 *   failure of the calling thread.
 * - Pointers named *_dev / device arrays are device (HBM) addresses; *_host are
 *   host addresses. All buffers are owned by the caller and only borrowed: the
 *   caller keeps them alive until the stream has passed the enqueued work. The
 *   library allocates no device memory.
 * - stream is a hipStream_t passed as void* (NULL = the default stream). Work is
 *   enqueued asynchronously; argument validation happens synchronously on the
 *   host before anything is enqueued, so a failed call enqueues nothing. Device
 *   faults surface at the caller's next synchronisation of that stream.
 * - One controlling thread; the library takes no locks.
 *
 * Linear-blocks. For a layer with E routed and S shared experts, block
 * i = 2*e + u, e in [0, E+S) (routed first), u = 0 for gate_up ([N=2I rows,
 * Kd=H]; rows 0..I-1 gate, rows I..2I-1 up) and u = 1 for down ([N=H, Kd=I]).
 * Supported bitwidths B_i = {3,...,8} for every block.
 *
 * Canonical bit-plane format (the interchange format mpb_pack_block reads):
 * planes[p][n][w], uint32, p = 0..7 with plane 0 the code's most significant
 * bit; bit j of word w holds element k = 32*w + j of row n. The b-bit index of
 * an element is formed from planes 0..b-1 (the top b planes, §2.2 and §3.1).
 * Canonical LUT of bitwidth b: [N][2^b] fp16 (one centroid table per row),
 * indexed by that b-bit index.
 */
#ifndef MPB_H
#define MPB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MPB_OK = 0,
    MPB_E_ARG = -1,          /* null pointer, bad enum, bad count */
    MPB_E_SHAPE = -2,        /* dimension not supported (see each call) */
    MPB_E_RANGE = -3,        /* block index i or bitwidth b out of range */
    MPB_E_NOT_RESIDENT = -4, /* bitwidth above the block's resident planes */
    MPB_E_WS = -5,           /* workspace too small */
    MPB_E_HIP = -6,          /* a HIP launch or API call failed */
    MPB_E_UNINIT = -7,       /* mpb_init has not bound a layer */
    MPB_E_BUSY = -8          /* a page transfer of the block is still in flight */
};

enum { MPB_PAGE_GPU = 0, MPB_PAGE_CPU = 1, MPB_PAGE_IN_TRANSFER = 2 }; /* page states */

enum { MPB_F16 = 0, MPB_BF16 = 1 }; /* activation dtypes */

typedef struct {
    int32_t H; /* hidden size, multiple of 64 */
    int32_t I; /* expert intermediate size, multiple of 64 */
    int32_t E; /* routed experts, 1..512 */
    int32_t S; /* shared (always-on) experts, 0..64 */
    int32_t K; /* experts per token, 1..min(E,16) */
} mpb_layer_desc;

/*
 * Bind a layer: its geometry and the weight page table of committed bitwidths
 * q_i (§3.1: one table row per linear-block; q_i is the bitwidth the serving
 * kernels read the block at). q_dev is a caller-owned device int32 array of
 * 2*(E+S) entries that the FFN kernels read; q_init_host (2*(E+S) values in
 * 3..8) is copied into it on `stream` and into the host mirror, and all planes
 * of every block are marked resident. `stream` becomes the stream on which
 * set_committed_bits enqueues its updates. Rebinding replaces the previous
 * layer. Errors: MPB_E_ARG (null pointer), MPB_E_SHAPE (geometry outside the
 * ranges above), MPB_E_RANGE (an initial q outside 3..8), MPB_E_HIP.
 */
int mpb_init(const mpb_layer_desc* d, int32_t* q_dev, const int32_t* q_init_host, void* stream);

/* Bytes of one packed plane page of an [N][Kd] block: N * ceil(Kd/128) * 16
 * (= N*Kd/8 when Kd is a multiple of 128; rows are padded to 128 elements). */
size_t mpb_plane_page_bytes(int N, int Kd);

/*
 * Packer (bit-plane layout for the kernels). Reads one block's canonical planes
 * canon_dev ([8][N][Kd/32] uint32, device) and writes 8 packed plane pages,
 * plane_pages_host[p] (host array of 8 device pointers, each
 * mpb_plane_page_bytes(N, Kd) bytes). Packed pages are plane-major, so a block
 * at bitwidth b is read through its first b pages only (§3.1: a b-bit block
 * consists of b bit-planes and the b-bit table). The packed layout inside a
 * page is private to this library. Needs N % 32 == 0 and Kd % 64 == 0, else
 * MPB_E_SHAPE. Does not need mpb_init.
 */
int mpb_pack_block(const uint32_t* canon_dev, int N, int Kd, uint32_t* const* plane_pages_host,
                   void* stream);

/*
 * Table images (§2.2: a b-bit weight is its b-bit index plus the b-bit lookup
 * table; §3.3: the fused kernel reads the table at the committed bitwidth).
 * moe_ffn reads every block's b-bit LUT from an image laid out the way its
 * kernels hold tables on chip, so that a workgroup loads its part with plain
 * copies. kind 0: a gate_up block (N = 2I rows: 0..I-1 gate, I..2I-1 up;
 * N % 128 == 0); kind 1: a down block (N = H rows; N % 64 == 0); N <= 131072;
 * b in 3..8.
 * mpb_table_image_bytes returns ceil(N/128) * 256 * 2^b, or MPB_E_ARG (bad
 * kind), MPB_E_RANGE (b) or MPB_E_SHAPE (N). mpb_pack_table reads the canonical
 * [N][2^b] fp16 LUT lut_dev and writes the image to image_dev (that many
 * bytes, device), enqueued on stream; same errors plus MPB_E_ARG for a null
 * pointer and MPB_E_HIP. The layout inside an image is private to this
 * library. Neither needs mpb_init.
 */
int64_t mpb_table_image_bytes(int kind, int N, int b);
int mpb_pack_table(int kind, const uint16_t* lut_dev, int N, int b, uint16_t* image_dev, void* stream);

/*
 * Router (§2.1: a learned gate scores all E experts per token; the K best are
 * run and weighted). X_dev: [T][H] activations of x_dtype (MPB_F16 or
 * MPB_BF16); W_router_dev: [E][H] fp32; bias_dev: [E] fp32 added to the
 * logits, or NULL. Logits are accumulated in fp64 (every product of an
 * activation and a router weight is exact in fp64) in a fixed order. Writes
 * topk_idx_dev [T][K] int32: the K largest exact logits in descending order,
 * ties to the lower expert index (the fp64 order is checked against a bound
 * on its rounding error; experts the bound cannot separate are ranked again
 * on their exact sums), and topk_w_dev [T][K] fp32 = softmax over all E
 * experts restricted to the K winners and renormalised (equal to a softmax
 * over the K winning fp64 logits).
 * ws_dev: device workspace of ws_bytes >= moe_route_workspace_bytes(T, E)
 * (fp64 logits, summed in up to 8 hidden-dimension parts for small batches,
 * and the norms that bound their rounding error; unused for batches of up to
 * 128 tokens with E * H <= 16384, whose logits stay on chip; contents not
 * preserved). Needs
 * 1 <= K <= min(E, 16), E <= 512, H a multiple of 64 up to 65536, T <= 2^20;
 * T == 0 is a no-op. Errors: MPB_E_ARG, MPB_E_SHAPE, MPB_E_WS, MPB_E_HIP.
 * Does not need mpb_init.
 */
size_t moe_route_workspace_bytes(int T, int E);
int moe_route(const void* X_dev, int x_dtype, const float* W_router_dev, const float* bias_dev,
              int T, int H, int E, int K, int32_t* topk_idx_dev, float* topk_w_dev, void* ws_dev,
              size_t ws_bytes, void* stream);

/*
 * Routing mass of a batch (§2.1, Eq. 1; the statistic the planner's hot and
 * cold buckets are built from, §3.2): mass_dev[e] = sum of topk_w over the
 * entries routed to expert e / sum of topk_w over all entries, for e < E, in
 * fp64 with a fixed summation order (deterministic). topk_idx_dev/topk_w_dev
 * are [T][K] as written by moe_route; ids outside [0, E) are ignored; an
 * empty batch gives zeros. Needs E <= 512, K <= min(E, 16), T <= 2^20.
 * Errors: MPB_E_ARG, MPB_E_SHAPE, MPB_E_HIP. Does not need mpb_init.
 */
int moe_routing_mass(const int32_t* topk_idx_dev, const float* topk_w_dev, int T, int E, int K,
                     double* mass_dev, void* stream);

/* Workspace bytes moe_ffn needs for T tokens of the bound layer (0 if unbound). */
size_t moe_ffn_workspace_bytes(int T);

/*
 * Fused MoE FFN of the bound layer (§3.3): groups the T tokens by expert,
 * runs gate_up + SwiGLU (h = SiLU(gate) * up) and the down projection of
 * every expert with tokens, and accumulates
 *   out[t] = sum_k topk_w[t][k] * FFN_{topk_idx[t][k]}(x_t) + sum_s FFN_{E+s}(x_t).
 * Each block's weights are dequantised on the fly from its first q_i packed
 * plane pages and its q_i-bit LUT, with q_i read from q_dev on the device.
 *   X_dev       [T][H] x_dtype activations
 *   topk_idx_dev/topk_w_dev  [T][K] as produced by moe_route; expert ids
 *               outside [0, E) contribute nothing
 *   planes_dev  device array of 2*(E+S)*8 device pointers: entry i*8 + p is
 *               plane page p of block i (written by mpb_pack_block). Only pages
 *               p < q_i are dereferenced.
 *   luts_dev    device array of 2*(E+S)*6 device pointers: entry i*6 + (b-3) is
 *               block i's b-bit table image (mpb_pack_table; kind 0 for even
 *               i, kind 1 for odd i). Only b == q_i is read.
 *   q_dev       the page table bound by mpb_init (MPB_E_ARG for any other);
 *               values 3..8
 *   out_dev     [T][H] fp32, overwritten
 *   ws_dev      workspace of ws_bytes >= moe_ffn_workspace_bytes(T)
 *   stream      the stream bound by mpb_init, where set_committed_bits
 *               writes q_i (so every launch is ordered with every commit, and
 *               page offloads wait for the launches that may read the pages),
 *               or a stream under graph capture (its kernels run when the
 *               graph is replayed; ordering replays against commits and page
 *               offloads is then the caller's part). Any other stream:
 *               MPB_E_ARG.
 * The kernels' on-chip table space is sized at enqueue time for the highest
 * bitwidth in the host mirror; a graph captured from this call must be
 * captured again after a block is raised above that bitwidth (its outputs
 * would otherwise be NaN, never silently wrong).
 * Results are deterministic for every T: the grouping counts with integer
 * atomics only, and every floating-point sum runs in a fixed order.
 * Errors: MPB_E_UNINIT, MPB_E_ARG, MPB_E_WS, MPB_E_HIP, and MPB_E_SHAPE when T
 * is too large for the layer (the kernels address the activations, T*H*2
 * bytes, and h, about 4*T*(K+S)*I bytes, with 32-bit offsets: each must stay
 * below 4 GiB; the launch grid must stay below 2^31 workgroups).
 */
int moe_ffn(const void* X_dev, int x_dtype, int T, const int32_t* topk_idx_dev,
            const float* topk_w_dev, const uint32_t* const* planes_dev,
            const uint16_t* const* luts_dev, const int32_t* q_dev, float* out_dev, void* ws_dev,
            size_t ws_bytes, void* stream);

/*
 * moe_ffn for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments, kernels and results as moe_ffn, with the workspace taken from a
 * device array that the library holds, 32 MiB per GPU, for the life of the
 * process (its address is looked up once per device, at mpb_init or at the
 * first call on that device). Allocates nothing itself; the caller still
 * passes inputs and outputs. Tokens whose workspace (moe_ffn_workspace_bytes
 * for bf16, slightly less for fp16) exceeds 32 MiB are refused with
 * MPB_E_WS: the limit is 292 tokens for a layer of H 2048, I 1408, 60 routed
 * + 4 shared experts, top-4, and 151 tokens for H 4096, I 14336, 8 experts,
 * top-2. Every call on one GPU shares that
 * GPU's array and leaves its contents behind; nothing in it needs to start at
 * zero. Calls that overlap on one GPU (on different streams, or from
 * different threads) race on the array and must be serialised by the caller.
 * Errors: as moe_ffn.
 */
int moe_ffn_static(const void* X_dev, int x_dtype, int T, const int32_t* topk_idx_dev,
                   const float* topk_w_dev, const uint32_t* const* planes_dev,
                   const uint16_t* const* luts_dev, const int32_t* q_dev, float* out_dev, void* stream);

/*
 * The whole layer in one launch (§3.3: routing, expert activation, down
 * projection and output accumulation in one fused kernel): moe_route followed
 * by moe_ffn, as one persistent kernel whose workgroups take units of work in
 * a fixed order (router logits, top-K, grouping, gate_up tiles, down tiles,
 * combine) and wait on device counters for the units they read from; a down
 * tile starts as soon as its own group's gate_up tiles are done. Results are
 * bit-identical to moe_route + moe_ffn on the same inputs (same arithmetic,
 * same order), except that for batches of up to 128 tokens with at most 16384
 * router weights moe_route sums each fp64 logit in another fixed order, which
 * can change the routing only where two logits lie within an fp64 ulp of a
 * tie or a weight within one of an fp32 rounding boundary. Arguments as for
 * those two calls; topk_idx_dev / topk_w_dev
 * receive the routing. ws_dev: at least moe_fused_workspace_bytes(T) bytes,
 * 256-byte aligned; its first moe_fused_counter_bytes() bytes are counters
 * that must be zero before the first call with this workspace (allocate it
 * zero-filled); every call leaves them zero again, so the workspace can be
 * reused, also by graph replays.
 * Calls sharing a workspace must not overlap. Every device-side wait is
 * bounded: a wait that runs out (only possible if the counters were not zero)
 * makes out NaN. Gate_up takes 32-token items (the decode configuration) for
 * every T. The stream rule is moe_ffn's. Errors: as moe_route and moe_ffn, plus MPB_E_ARG for a misaligned
 * workspace.
 */
size_t moe_fused_counter_bytes(void);
size_t moe_fused_workspace_bytes(int T);
int moe_fused(const void* X_dev, int x_dtype, int T, const float* W_router_dev, const float* bias_dev,
              int32_t* topk_idx_dev, float* topk_w_dev, const uint32_t* const* planes_dev,
              const uint16_t* const* luts_dev, const int32_t* q_dev, float* out_dev, void* ws_dev,
              size_t ws_bytes, void* stream);

/*
 * Commit bitwidth b for linear-block i (§3.1 and §3.3: the planner lowers or
 * raises q_i at a safe boundary; a reload raises q_i only once its pages are
 * GPU-resident). Validates 0 <= i < 2*(E+S), b in 3..8 and that planes 0..b-1
 * of the block are GPU-resident (a reload whose copies have not completed
 * leaves its pages in transfer, and the commit is refused until they have:
 * MPB_E_NOT_RESIDENT). Then updates the host mirror and enqueues the device
 * write of q_dev[i] on the bound stream: FFN launches enqueued before it read
 * the old value, later ones the new value. Errors: MPB_E_UNINIT, MPB_E_RANGE,
 * MPB_E_NOT_RESIDENT, MPB_E_HIP.
 */
int set_committed_bits(int i, int b);

/*
 * Weight bytes the committed bitwidths hold (§3.1, Eq. 3: M_i^b counts the b
 * bit-planes and the b-bit LUT of block i): sum over blocks of
 * N_i*Kd_i*q_i/8 + N_i*2^q_i*2, from the host mirror. touched_host, if not
 * NULL, is a host array of 2*(E+S) flags restricting the sum. Returns the byte
 * count, or MPB_E_UNINIT.
 */
int64_t mpb_committed_bytes(const uint8_t* touched_host);

/* Host mirror of q_i (test and planner use); MPB_E_UNINIT / MPB_E_RANGE. */
int mpb_get_committed_bits(int i);

/*
 * Test export: dequantise one block through the same device index assembly and
 * LUT lookup the FFN kernels use. pages_host: host array of b device pointers
 * (packed plane pages 0..b-1); lut_b_dev: canonical [N][2^b] fp16 LUT; writes
 * out_f16_dev [N][Kd] fp16 in canonical element order. Shapes as for
 * mpb_pack_block; b in 3..8 else MPB_E_RANGE.
 */
int mpb_dequant_block(const uint32_t* const* pages_host, const uint16_t* lut_b_dev, int N, int Kd,
                      int b, uint16_t* out_f16_dev, void* stream);

/*
 * The same dequantisation (§3.1, Eq. 2) read through a table image
 * (mpb_pack_table of kind `kind` for this block, b bits, image_dev on the
 * device) the way the FFN kernels stage and index it: a check that an image
 * holds every table entry where those kernels look it up. Writes out_f16_dev
 * [N][Kd] fp16 in canonical element order. Shapes as for mpb_table_image_bytes
 * (N % 128 == 0 for kind 0, N % 64 == 0 for kind 1) and Kd % 64 == 0;
 * MPB_E_ARG for a bad kind or a null pointer,
 * MPB_E_RANGE (b), MPB_E_SHAPE, MPB_E_HIP.
 */
int mpb_dequant_block_image(const uint32_t* const* pages_host, const uint16_t* image_dev, int kind, int N,
                            int Kd, int b, uint16_t* out_f16_dev, void* stream);

/*
 * Page movement (§3.1 after Eq. 3, §3.3 "Asynchronous Page Movement",
 * Figure 4: an offload first lowers q_i, then moves the pages above it to CPU
 * memory; a reload first moves the pages back and raises q_i only once they
 * are GPU-resident). A weight page is one bit-plane with its table state
 * (§3.1): page p (0..7) of block i is plane page p and, for p >= 2, the table
 * image of bitwidth p + 1 (the table a block reads once it uses p + 1 planes),
 * so a block with r resident pages can run at any q_i <= r. Each page is in
 * one state: MPB_PAGE_GPU (p below the block's resident count),
 * MPB_PAGE_IN_TRANSFER (a copy is enqueued and not known to have completed)
 * or MPB_PAGE_CPU. The library only enqueues copies and tracks states; the
 * caller owns every buffer.
 *
 * mpb_offload_pages(i, r, ...): needs q_i <= r (else MPB_E_NOT_RESIDENT:
 * lower q_i with set_committed_bits first). Enqueues on copy_stream the
 * copies of the resident pages p = r..7 to host memory: plane page p
 * (mpb_plane_page_bytes(N, Kd) bytes) from dev_planes[p] to host_planes[p],
 * table image p + 1 (mpb_table_image_bytes(i % 2, N, p + 1) bytes) from
 * dev_tables[p - 2] to host_tables[p - 2]. The copies start after every
 * launch enqueued on the bound stream before the last lowering of q_i (the
 * only launches that may read those pages). The pages are IN_TRANSFER at once
 * (commits above r are refused from now on) and CPU when the copies have
 * completed; from then on no FFN launch reads them and the caller may reuse
 * their device memory. No-op if no page above r is resident.
 * mpb_reload_pages(i, r, ...): enqueues on copy_stream the copies of the
 * non-resident pages p < r from host memory into the caller's device buffers
 * dev_planes[p] / dev_tables[p - 2] (if these moved, the caller also writes
 * their addresses into the pointer arrays it passes to moe_ffn). They are
 * IN_TRANSFER until the copies have completed, then GPU, and only then may
 * q_i be raised to r. No-op if pages 0..r-1 are already resident.
 * dev_planes / host_planes: host arrays of 8 pointers (entry p: plane page
 * p); dev_tables / host_tables: host arrays of 6 pointers (entry b - 3: the
 * table image of bitwidth b). Only the entries of the pages that move are
 * read and must be non-NULL. Host buffers should be pinned (hipHostMalloc)
 * for the copies to be asynchronous. copy_stream: a hipStream_t other than
 * the bound one, so the copies overlap the layer's kernels. A block has at
 * most one transfer in flight: MPB_E_BUSY otherwise. States are refreshed by
 * polling the transfer's completion (never blocking) in every call that
 * reads them.
 * Errors: MPB_E_UNINIT, MPB_E_RANGE (i, or r outside 3..8), MPB_E_ARG (a
 * needed pointer is NULL), MPB_E_NOT_RESIDENT, MPB_E_BUSY, MPB_E_HIP.
 */
int mpb_offload_pages(int i, int r, void* const* host_planes, const uint32_t* const* dev_planes,
                      void* const* host_tables, const uint16_t* const* dev_tables, void* copy_stream);
int mpb_reload_pages(int i, int r, const void* const* host_planes, uint32_t* const* dev_planes,
                     const void* const* host_tables, uint16_t* const* dev_tables, void* copy_stream);

/* State of page p (0..7) of block i: MPB_PAGE_*, or MPB_E_UNINIT /
 * MPB_E_RANGE / MPB_E_HIP (the transfer's copy stream reported a failure). */
int mpb_page_state(int i, int p);

/* Number of GPU-resident pages of block i (3..8; pages 0..n-1 are resident),
 * or MPB_E_UNINIT / MPB_E_RANGE. */
int mpb_get_resident_planes(int i);

/*
 * Test hook: declare how many of block i's planes are GPU-resident (3..8)
 * without moving anything; set_committed_bits then refuses b > r. Lowering r
 * below the committed q_i is refused with MPB_E_NOT_RESIDENT (offload lowers
 * q_i first), and any change while a transfer is in flight with MPB_E_BUSY.
 * MPB_E_UNINIT / MPB_E_RANGE.
 */
int mpb_set_resident_planes(int i, int r);

/*
 * Planner step (§3.2, Algorithm 1; Eqs. 3-8), host only: turns KV-cache
 * pressure into a byte target D (Eq. 7), scores one-bit reductions of routed
 * linear-blocks by predicted damage (Eq. 4 global damage, Eq. 5-6 prompt
 * residual, Eq. 8 with the routing bucket's multiplier) per released byte
 * (Eq. 3), greedily builds one candidate plan per bitwidth-floor stage, keeps
 * the newest plan of every stage in the queue, and when pressure is triggered
 * selects the page-movement plan {(i, q_i -> d_i, Delta_i)}.
 * Readings of the steps the pages leave open:
 *  - a step lowers one block by one bit; a block's steps are taken in order;
 *    GreedySelect repeatedly takes the available step with the smallest
 *    damage / released bytes (ties to the lower block index) until the
 *    released bytes reach D;
 *  - stage s allows block i down to max(stage_floor[s], floor of i's routing
 *    bucket); relaxing the depth cap is moving to the next stage;
 *  - SelectBestPlan: the first stage whose plan reaches D, else the plan that
 *    releases the most bytes (the largest safe reduction), ties to the earlier
 *    stage;
 *  - pressure is triggered when F_blk <= T_blk; D uses F_blk - P_blk (free
 *    blocks after the pending KV growth);
 *  - routing buckets: experts sorted by routing mass, hottest first (ties to
 *    the lower index); bucket k ends at rank ceil(bucket_frac[k] * E);
 *  - candidates are routed blocks whose pages may move (movable_host[i] != 0,
 *    or every routed block if movable_host is NULL); shared experts' blocks
 *    never change.
 * Floating-point evaluation order is fixed (Eq. 5 summed left to right, eta
 * through the C library's exp, damage sums in step order), so a plan is
 * reproducible bit for bit.
 */
typedef struct {
    int32_t n_buckets;         /* 1..8 */
    double bucket_frac[8];     /* cumulative share of experts per bucket, increasing, last 1.0 */
    double mu[8];              /* damage multiplier per bucket, > 0 */
    int32_t floor[8];          /* bitwidth floor per bucket, 3..8 */
    int32_t n_stages;          /* 1..6 */
    int32_t stage_floor[6];    /* global floor per stage, 3..8, strictly decreasing */
    double eps;                /* damage floor of Eq. 8, > 0 */
    double alpha;              /* strength of Eq. 6 */
    double rho_min, rho_max;   /* clip range of Eq. 6, rho_min <= rho_max */
    /* Eq. 5-6 heads per block type u (0 gate_up, 1 down) and one-bit
     * transition b -> b-1, b = 4..8 at index b - 4 */
    double head_w[2][5][3];
    double head_a[2][5];
    double head_c[2][5];       /* confidence */
    int64_t T_blk;             /* free-block threshold (Eq. 7) */
    int64_t F_blk;             /* current free KV blocks */
    int64_t P_blk;             /* pending KV growth in blocks (0: Eq. 7 as printed) */
    int64_t B_kv;              /* bytes of one KV block */
} mpb_planner_params;

typedef struct {
    int32_t i;                 /* linear-block */
    int32_t from, to;          /* q_i -> d_i */
    int64_t delta;             /* M_i^{from} - M_i^{to} (Eq. 3) */
    double damage;             /* sum of the predicted damage of its steps */
} mpb_plan_entry;

typedef struct {
    int64_t D;                 /* byte target (Eq. 7) */
    int32_t triggered;         /* 1 if pressure is triggered */
    int32_t stage;             /* stage of the selected plan, -1 if not triggered */
    int32_t n_plan;            /* entries written to plan_host */
    int32_t pad;
    int64_t released;          /* sum of delta over the selected plan */
    double damage;             /* sum of damage over the selected plan (entry order) */
    int64_t stage_released[6]; /* per stage plan in the queue */
    double stage_damage[6];
} mpb_plan_summary;

/*
 * mpb_plan_step(d, q_host, movable_host, sens_host, mass_host, phi_host, prm,
 *               queue_host, plan_host, summary):
 *   d            layer geometry (as for mpb_init; no layer needs to be bound)
 *   q_host       [2(E+S)] committed bitwidths (3..8)
 *   movable_host [2(E+S)] flags or NULL
 *   sens_host    [2(E+S)][6] s_i^b for b = 3..8 (Eq. 4)
 *   mass_host    [E] routing mass (Eq. 1, e.g. from moe_routing_mass)
 *   phi_host     [2(E+S)][3] routed-input features (Eq. 5)
 *   queue_host   out: [n_stages][2(E+S)] desired bitwidths of each stage's
 *                plan (the refreshed plan queue); may be NULL
 *   plan_host    out: up to 2(E+S) entries, ascending i, only when triggered
 *   summary      out
 * All pointers are host memory owned by the caller. Does not touch the GPU.
 * Errors: MPB_E_ARG (null pointer, parameter out of its range),
 * MPB_E_SHAPE (geometry), MPB_E_RANGE (a q outside 3..8).
 */
int mpb_plan_step(const mpb_layer_desc* d, const int32_t* q_host, const uint8_t* movable_host,
                  const double* sens_host, const double* mass_host, const double* phi_host,
                  const mpb_planner_params* prm, int32_t* queue_host, mpb_plan_entry* plan_host,
                  mpb_plan_summary* summary);

/*
 * Profiling hook: with n == 5 or 7, every following moe_ffn records
 * events_host[0..n-1] (host array of hipEvent_t handles, caller-created) on
 * its stream: 0 before the grouping kernels, 1 and 2 at the start and end of
 * the gate_up kernel (recorded by its launch, so 1 -> 2 is the kernel alone
 * and 0 -> 1 includes the dispatch of gate_up), 3 before the combine and 4
 * after it, and with n == 7, 5 and 6 at the start and end of the down kernel
 * (recorded by its launch), so the caller can time each phase with
 * hipEventElapsedTime. n == 0 turns recording off. The handles are borrowed
 * until the hook is changed. MPB_E_ARG for any other n or a null handle.
 */
int mpb_set_kernel_events(void* const* events_host, int n);

/* Message of the calling thread's last failure ("" if none). */
const char* mpb_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MPB_H */
