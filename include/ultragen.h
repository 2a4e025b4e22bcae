/*
 * ultragen.h -- C ABI of the MI355X (gfx950) hierarchical local attention
 * library: window-first permutation, 2D axial RoPE with scaled low-resolution
 * positions, one composite-masked attention forward, inverse permutation.
 *
 * The method is UltraGen's ("UltraGen: Efficient Ultra-High-Resolution Image
 * Generation with Hierarchical Local Attention"; papernotes.org notes,
 * sections 关键设计 1-3, and the gist.science summary, section 2.A-2.B).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every function is extern "C", never throws, never aborts, and returns a
 *    ug_status.  Arguments are validated before any HIP call is made; on
 *    failure nothing is launched and ug_last_error() holds a message
 *    (thread-local, valid until the next call on the same thread).
 *  - Tensors Q, K, V, O are device pointers to [B, L, Hh, D] contiguous
 *    arrays (D innermost), element type = the plan's dtype (fp32 or bf16),
 *    16-byte aligned.  Rows of one sequence are [text T | HR N | LR N_lr]
 *    (the joint sequence [C_T; X; X_lr] of 关键设计 3).
 *      raster layout:   HR row T + r*W + c holds grid token (r, c);
 *                       LR row T + N + m*w + n holds LR token (m, n).
 *      permuted layout: HR rows in window-first order (windows row-major,
 *                       tokens row-major inside a window; partial windows at
 *                       the bottom/right edges of a ragged grid, no padding);
 *                       text rows keep their places; LR rows keep theirs
 *                       unless lr_mode = 1 (then window-first as well).
 *  - The caller owns every tensor and the workspace; the plan owns its own
 *    device tables.  No entry point allocates device memory except ug_plan.
 *  - Launches are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Device faults surface at the caller's next synchronisation.
 *    A plan's tables are immutable after creation and a plan may serve
 *    several streams at once.  The attention forward and the dQ pass of
 *    ug_attn_bwd run as persistent grids whose workgroups take query tiles
 *    from work queues through atomic cursors that the plan owns: each such
 *    launch takes the next of 64 cursor slots and leaves it cleared when it
 *    ends, so at most 64 of them (ug_attn_bwd counts one) may be in flight
 *    with one plan at the same time.  A launch captured in a HIP graph keeps
 *    its slot: replays of that graph must not overlap one another.
 */
#ifndef ULTRAGEN_H
#define ULTRAGEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ug_status {
  UG_OK = 0,
  UG_ERR_INVALID_ARGUMENT = 1,  /* bad descriptor, pointer, alignment or aliasing */
  UG_ERR_UNSUPPORTED = 2,       /* valid request the GPU kernels do not cover */
  UG_ERR_OUT_OF_MEMORY = 3,     /* host or device allocation failed (ug_plan only) */
  UG_ERR_HIP = 4,               /* a HIP runtime call or kernel launch failed */
  UG_ERR_INTERNAL = 5
} ug_status;

typedef enum ug_dtype { UG_F32 = 0, UG_BF16 = 1 } ug_dtype;

/* ug_desc.flags */
#define UG_PLAN_HOST_ONLY 1 /* build host tables only: no HIP call; only
                               ug_plan_info / ug_plan_export / ug_plan_free
                               may then be used */
#define UG_PLAN_NO_LR 2     /* no LR tokens (lr_h and lr_w must then be 0) */

/*
 * Geometry of one attention layer.
 *  - hr_h x hr_w: HR latent token grid (关键设计 1: X in R^{H x W}).
 *  - lr_h x lr_w: LR guidance grid (关键设计 2: X_lr in R^{h x w}).  0 x 0
 *    means the grid the scaling implies, ceil(hr_h/rho) x ceil(hr_w/rho)
 *    (one LR token per rho x rho block of HR tokens); flag UG_PLAN_NO_LR
 *    (with 0 x 0) means no LR tokens; exactly one of them 0 is an error.
 *    LR token (m, n) takes RoPE position (rho*m, rho*n) (关键设计 2, the
 *    coordinate-scaling equation).  ug_plan_info and the exports report the
 *    grid the plan uses.
 *  - window: l, the window side in tokens (l = 16 in 关键设计 1).  Windows
 *    of more than 256 tokens are split into several query tiles.
 *  - radius: HR queries see HR keys whose window is within Chebyshev
 *    distance `radius` of their own (1 = own + adjacent windows, 3x3).
 *  - lr_mode: which LR tokens an HR query sees.  0 = all of them (the LR
 *    latent as one global anchor set, gist.science summary 2.B).  1 = only
 *    the "corresponding" anchors of 关键设计 2: LR token (m, n) belongs to the
 *    window containing its scaled position (rho*m, rho*n), and an HR query
 *    sees the LR tokens of the windows within `radius` of its own.  With
 *    lr_mode 1 the permuted layout also orders the LR rows window-first (by
 *    that window, then row-major); LR tokens outside the window grid go last.
 *  - rope_theta: base of the axial RoPE frequencies omega_k =
 *    theta^(-2k/(D/2)); dims [0, D/2) are rotated by the row position,
 *    [D/2, D) by the column position, pairs (2k, 2k+1).
 *  - GPU kernels support head_dim 64 or 128; dtype UG_BF16 or UG_F32.
 */
typedef struct ug_desc {
  int32_t batch;
  int32_t heads;
  int32_t head_dim;
  int32_t hr_h, hr_w;
  int32_t lr_h, lr_w;
  int32_t n_text;
  int32_t window;
  int32_t radius;
  int32_t rho;
  int32_t dtype; /* ug_dtype */
  int32_t flags; /* UG_PLAN_* */
  int32_t lr_mode; /* 0: HR queries see all LR tokens; 1: corresponding LR only */
  double rope_theta;
} ug_desc;

typedef struct ug_info {
  int64_t seq_len;             /* L = T + N + N_lr */
  int64_t n_hr;                /* N = hr_h * hr_w */
  int64_t n_lr;                /* lr_h * lr_w */
  int64_t n_text;              /* T */
  int32_t grid_y, grid_x;      /* windows per column / row: ceil(H/l), ceil(W/l) */
  int32_t n_windows;           /* grid_y * grid_x */
  int32_t max_neighbours;      /* most windows any window sees */
  int64_t n_neighbour_entries; /* length of the exported neighbour list */
  int64_t pairs_per_head;      /* exact number of allowed (query, key) pairs */
  double eff_flops;            /* 4 * D * pairs_per_head * heads * batch */
  int64_t workspace_bytes;     /* bytes ug_attn_fwd needs as workspace (0 today) */
  int64_t attn_tasks;          /* query tiles per (batch, head) */
  int64_t attn_blocks;         /* items of the attention's 8 per-XCD work queues (one per query
                                  tile and batch*head, plus idle padding); ug_attn_fwd launches
                                  min(compute units, attn_blocks) persistent workgroups */
  int64_t attn_key_tiles;      /* 64-key tiles processed per (batch, head) */
  int64_t rope_positions;      /* rows of the RoPE cos/sin table */
  int64_t bwd_workspace_bytes; /* bytes ug_attn_bwd needs as workspace */
  int64_t bwd_key_tasks;       /* key tiles per (batch, head) of the dK/dV pass */
  int64_t bwd_blocks;          /* workgroups one dK/dV pass launches */
  int64_t attn_ranges;         /* key ranges of all query tiles (ug_plan_export_blocks) */
  int64_t bwd_key_ranges;      /* query ranges of all key tiles */
  int64_t bwd_mask_words;      /* 64-bit range masks of the masked key tiles */
} ug_info;

typedef struct ug_plan_s* ug_plan_t;

/*
 * ug_plan: validate `desc`, build the host tables (window-first permutation
 * and inverse, window offsets, window neighbourhoods, the per-query-tile key
 * range list and workgroup order, RoPE cos/sin table computed in double and
 * stored as float) and, unless UG_PLAN_HOST_ONLY, upload them to the current
 * HIP device and allocate the attention's zeroed work-queue cursors (4 KiB)
 * there, with the events that order their reuse and the backward's second
 * stream (synchronous).  The window-first order is 关键设计 1's regrouping
 * of tokens window by window; the neighbourhood is its adjacent-window
 * interaction.  On success *out owns everything; free it with ug_plan_free
 * once no launched work still uses it.
 */
ug_status ug_plan(const ug_desc* desc, ug_plan_t* out);
ug_status ug_plan_free(ug_plan_t plan);
ug_status ug_plan_info(ug_plan_t plan, ug_info* out);

/*
 * ug_plan_export: host copies of the plan's integer tables, for inspection
 * and bit-exact tests.  Any pointer may be NULL to skip that table.
 *  perm    int32[N]            perm[j] = raster HR index of window-first slot j
 *  win_off int32[n_windows+1]  window w occupies slots [win_off[w], win_off[w+1])
 *  nbr     int32[n_neighbour_entries]  windows (ascending) each window sees
 *  nbr_off int32[n_windows+1]  window w's list is nbr[nbr_off[w] .. nbr_off[w+1])
 */
ug_status ug_plan_export(ug_plan_t plan, int32_t* perm, int32_t* win_off, int32_t* nbr,
                         int32_t* nbr_off);

/*
 * ug_plan_export_lr: the LR tables (either pointer may be NULL).
 *  lr_perm    int32[n_lr]           raster LR index held by LR slot i of the
 *                                   permuted layout (the identity when
 *                                   lr_mode = 0)
 *  lr_win_off int32[n_windows + 2]  LR slots [lr_win_off[w], lr_win_off[w+1])
 *                                   hold window w's anchors (lr_mode = 1
 *                                   order); entries n_windows .. n_windows+1
 *                                   bound the out-of-grid tail
 */
ug_status ug_plan_export_lr(ug_plan_t plan, int32_t* lr_perm, int32_t* lr_win_off);

/*
 * ug_plan_export_queues: the per-XCD work queues (either pointer may be
 * NULL), as (task, batch*head) pairs; task = -1 marks padding.
 *  attn_items int32[2 * info.attn_blocks]  query tiles of the attention
 *                                          forward and of the backward's dQ pass
 *  bwd_items  int32[2 * info.bwd_blocks]   key tiles of the dK/dV pass
 * Item k*8 + x is the k-th item of XCD x's queue.  Each queue holds its
 * items first and padding only after them, which the persistent grids rely
 * on (a cursor on padding means that queue is empty).
 */
ug_status ug_plan_export_queues(ug_plan_t plan, int32_t* attn_items, int32_t* bwd_items);

/*
 * ug_plan_export_blocks: the block lists the attention kernels walk, for
 * bit-exact tests of the mask they encode (关键设计 1-2: windows, adjacent
 * windows, text and LR anchors).  Any pointer may be NULL to skip a table.
 * Rows are rows of the permuted sequence; every list is per (batch, head)
 * and the same for all of them.
 *  q_tiles    int32[4 * info.attn_tasks]   query tile t: query rows
 *                                          [q_tiles[4t], q_tiles[4t+1]) see
 *                                          the key ranges q_tiles[4t+2] ..
 *                                          q_tiles[4t+3]-1 of k_ranges
 *  k_ranges   int32[2 * info.attn_ranges]  range r: key rows [k_ranges[2r],
 *                                          k_ranges[2r+1])
 *  k_tiles    int32[4 * info.bwd_key_tasks] key tile u of the backward's
 *                                          dK/dV pass: key rows [k_tiles[4u],
 *                                          k_tiles[4u+1]) and the query ranges
 *                                          k_tiles[4u+2] .. k_tiles[4u+3]-1
 *                                          of q_ranges
 *  q_ranges   int32[2 * info.bwd_key_ranges] range r: query rows
 *                                          [q_ranges[2r], q_ranges[2r+1])
 *  mask_off   int32[info.bwd_key_tasks]    -1: every key of tile u sees all
 *                                          of the tile's query ranges; else
 *                                          key row k_tiles[4u] + j sees its
 *                                          tile's range number b iff bit b of
 *                                          masks[mask_off[u] + j] is set
 *  masks      uint64[info.bwd_mask_words]
 * The union of a query row's ranges is exactly the set of keys it attends
 * to, and the union of a key row's (masked) ranges exactly the queries that
 * attend to it.
 */
ug_status ug_plan_export_blocks(ug_plan_t plan, int32_t* q_tiles, int32_t* k_ranges, int32_t* k_tiles,
                                int32_t* q_ranges, int32_t* mask_off, uint64_t* masks);

/*
 * ug_permute: x_perm = x_raster with HR rows gathered into window-first
 * order (关键设计 1; gist.science summary 2.A, window-first token
 * permutation); text and LR rows copied unchanged.  Out of place:
 * x_raster == x_perm (or any overlap) is UG_ERR_INVALID_ARGUMENT.
 * ug_unpermute is the exact inverse (bit copies both ways).
 */
ug_status ug_permute(ug_plan_t plan, const void* x_raster, void* x_perm, void* stream);
ug_status ug_unpermute(ug_plan_t plan, const void* x_perm, void* x_raster, void* stream);

/*
 * ug_rope2d: in place on permuted Q and K, rotate every HR and LR row by its
 * 2D position (HR: grid (r, c); LR: (rho*m, rho*n), 关键设计 2); text rows are
 * left unchanged (position (0, 0)).  Math in fp32, bf16 results rounded to
 * nearest even.  q_perm and k_perm must not overlap.
 */
ug_status ug_rope2d(ug_plan_t plan, void* q_perm, void* k_perm, void* stream);

/*
 * ug_attn_fwd: O = softmax(Q K^T / sqrt(D) + M) V per (batch, head) on
 * permuted, rotated Q and K and permuted V (关键设计 3's joint attention over
 * [C_T; X; X_lr]).  M is the composite mask of 关键设计 2: a text query sees
 * text and HR keys; an HR query sees text, the HR keys of its own and
 * adjacent windows, and all LR keys (lr_mode 0) or the LR anchors of those
 * same windows (lr_mode 1); an LR query sees LR and text.  Masked keys are
 * excluded (additive -inf).  O is written in the permuted layout.  bf16: bf16
 * MFMA products, fp32 softmax and accumulation, O rounded to nearest even;
 * fp32: fp32 MFMA throughout.  `workspace` is part of the boundary's
 * signature but not read: info.workspace_bytes is 0 for every plan (the
 * kernels' work-queue cursors live in the plan), so it may be NULL.  o must
 * not overlap q, k or v.
 */
ug_status ug_attn_fwd(ug_plan_t plan, const void* q, const void* k, const void* v, void* o,
                      void* workspace, void* stream);

/*
 * Fused forms of the same path (one fewer HBM pass each; results are
 * bit-identical to the separate calls):
 *
 * ug_permute_rope: q_perm/k_perm = ug_permute of q_raster/k_raster followed
 * by ug_rope2d, in one read and one write of Q and K (window-first order of
 * 关键设计 1 and the scaled-position RoPE of 关键设计 2).  Out of place: no
 * output may overlap an input, and q_perm must not overlap k_perm.
 *
 * ug_attn_fwd_raster: ug_attn_fwd with the output written in the raster
 * layout, i.e. ug_attn_fwd followed by ug_unpermute, without the extra pass.
 * Same arguments and rules as ug_attn_fwd; o_raster must not overlap q, k, v.
 */
ug_status ug_permute_rope(ug_plan_t plan, const void* q_raster, const void* k_raster, void* q_perm,
                          void* k_perm, void* stream);
ug_status ug_attn_fwd_raster(ug_plan_t plan, const void* q, const void* k, const void* v, void* o_raster,
                             void* workspace, void* stream);

/*
 * Training path.  UltraGen fine-tunes its LR branch through the joint
 * attention (关键设计 3 and the training section: LoRA on the LR Q, K, V
 * projections, flow-matching loss), so the layer needs its gradients.
 * ug_attn_bwd works on bf16 plans with head_dim 64 or 128 (otherwise
 * UG_ERR_UNSUPPORTED); ug_attn_fwd_lse and ug_rope2d_bwd accept every plan
 * their forward counterparts accept.
 *
 * ug_attn_fwd_lse: ug_attn_fwd that also writes lse[B][Hh][L] (float32,
 * 4-byte aligned, rows in the permuted order): the natural log of each row's
 * softmax denominator, log(sum over allowed j of exp(q.k_j / sqrt(D))).
 * lse must not overlap q, k, v or o.
 *
 * ug_attn_bwd: gradients of the same attention, in the permuted layout, given
 * dO (d_o), the forward's output o and lse:
 *   dq, dk = dL/dQ, dL/dK with respect to the rotated (ug_rope2d'ed) Q and
 *   K; dv = dL/dV.  With P = exp(S - lse), S = QK^T/sqrt(D) over the allowed
 *   keys, Delta_i = dO_i . O_i and dS = P * (dO V^T - Delta):
 *   dq = dS K / sqrt(D), dk = dS^T Q / sqrt(D), dv = P^T dO.
 * `workspace` (caller-owned, 16-byte aligned, info.bwd_workspace_bytes) holds
 * per-row statistics; its contents need no initialisation.  Outputs are
 * written in full (no accumulation into them) and must not overlap each
 * other, the inputs, lse or the workspace.  The result does not depend on
 * scheduling (no atomics).  Products in bf16 MFMA with fp32 accumulation;
 * P and dS are rounded to bf16 as MFMA operands.  The dK/dV pass runs on a
 * stream the plan owns, beside the dQ pass on `stream`, forked from and
 * joined back to `stream` by events: work queued on `stream` afterwards sees
 * all three gradients, as with a single stream.  Calls on one plan from
 * several host threads are serialised while they queue their work; stream
 * capture is refused (UG_ERR_UNSUPPORTED) before anything is queued.
 *
 * ug_rope2d_bwd: in place on permuted dq and dk, the transpose of
 * ug_rope2d's rotation (each pair turns by the negated angle), which maps
 * gradients with respect to the rotated Q, K to gradients with respect to
 * Q, K.  Same arguments and rules as ug_rope2d.
 *
 * ug_permute_rope_bwd: the transpose of ug_permute_rope, for the gradients:
 * dq_raster/dk_raster = ug_rope2d_bwd of dq_perm/dk_perm followed by
 * ug_unpermute, in one read and one write (bit-identical to the two calls).
 * The inputs are not modified.  Out of place: no output may overlap an
 * input, and dq_raster must not overlap dk_raster.  Any plan ug_rope2d
 * accepts.
 *
 * A layer's backward in raster layout is then: ug_permute(dO) ->
 * ug_attn_bwd -> ug_permute_rope_bwd(dq, dk) and ug_unpermute(dv) (or,
 * unfused, ug_rope2d_bwd(dq, dk) -> ug_unpermute of dq, dk and dv).
 */
ug_status ug_attn_fwd_lse(ug_plan_t plan, const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, void* stream);
ug_status ug_attn_bwd(ug_plan_t plan, const void* q, const void* k, const void* v, const void* o,
                      const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                      void* stream);
ug_status ug_rope2d_bwd(ug_plan_t plan, void* dq_perm, void* dk_perm, void* stream);

/*
 * ug_attn_bwd_noalloc: ug_attn_bwd for callers that cannot allocate device
 * memory (tight serving or training loops, harnesses that forbid hipMalloc):
 * the same kernels and results, with the per-row statistics kept in a
 * library-owned scratch array instead of a caller workspace.  It calls no
 * allocating routine.
 *  - The scratch is 64 MiB (67108864 bytes) per GPU, held from the first
 *    call on that GPU until the process ends; a plan whose
 *    info.bwd_workspace_bytes exceeds it gets UG_ERR_UNSUPPORTED (use
 *    ug_attn_bwd).  4K with 24 heads needs 13.5 MB, 8K 53.6 MB.
 *  - Every call on one GPU uses that GPU's one scratch: calls that overlap in
 *    time on one GPU (other streams, other threads, other plans) race and
 *    must be serialised by the caller.  Nothing in it needs clearing: each
 *    call writes every statistic it reads.
 *  - Same arguments and rules as ug_attn_bwd otherwise.
 */
ug_status ug_attn_bwd_noalloc(ug_plan_t plan, const void* q, const void* k, const void* v, const void* o,
                              const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* stream);
ug_status ug_permute_rope_bwd(ug_plan_t plan, const void* dq_perm, const void* dk_perm, void* dq_raster,
                              void* dk_raster, void* stream);

/*
 * Guidance-weighted warm start (关键设计 4; gist.science summary 2.C): the HR
 * sampler starts at normalised time alpha = t/T from
 *   x_hr = alpha * noise + (1 - alpha) * Y,
 *   Y = U + sharpen * (U - B*U),  U = bilinear upsampling of x_lr,
 * where LR sample (m, n) sits at HR (rho*m, rho*n) (the coordinate map of
 * 关键设计 2; past the last LR row/column the last sample's value is kept),
 * and B is the 3x3 binomial blur ([1 2 1]/4 in each direction, edges
 * replicated).  The pages name interpolation and sharpening without fixing
 * them; these are the plainest linear choices.  noise is the caller's
 * Gaussian draw X_T (the library draws no random numbers).
 *  - x_lr:  [batch, lr_h, lr_w, channels], noise and x_hr: [batch, hr_h,
 *    hr_w, channels]; contiguous, channels innermost (latent tokens in raster
 *    order, as the attention's HR rows), dtype fp32 or bf16, 16-byte aligned;
 *    channels a multiple of 4 (fp32) or 8 (bf16).
 *  - fp32 arithmetic, one RNE rounding of the bf16 output.
 *  - x_hr may be noise itself (in place); any other overlap is an error.
 *  - Stateless: no plan; nothing is allocated.
 */
typedef struct ug_warm_desc {
  int32_t batch;
  int32_t hr_h, hr_w;
  int32_t lr_h, lr_w;
  int32_t channels;
  int32_t rho;
  int32_t dtype;  /* ug_dtype */
  float alpha;    /* t / T, in [0, 1] */
  float sharpen;  /* unsharp-mask strength, >= 0 (0: none) */
} ug_warm_desc;

ug_status ug_warm_start(const ug_warm_desc* desc, const void* x_lr, const void* noise, void* x_hr, void* stream);

const char* ug_status_str(ug_status s);
const char* ug_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ULTRAGEN_H */
