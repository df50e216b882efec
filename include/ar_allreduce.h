/*
 * ar_allreduce.h -- C ABI of the MI355X sum all-reduce over R rank buffers.
 *
 * One process, one GPU.  R "ranks" are R buffers in the GPU's HBM that stand
 * in for the peer memory a memory-mapped channel would expose (the
 * MemoryChannel of "MSCCL++：让 GPU 通信像 CUDA 一样可编程",
 * infinitensor.com/news/50, section "MemoryChannel": GPU threads load and store
 * the other GPU's memory directly).  One call reduces the R send buffers
 * element by element and writes the sum to all R receive buffers.
 *
 * The call is shaped like the NCCL-compatible collective that the same page
 * describes under "第一层：Collective API" (mscclppAllReduce as a drop-in for
 * ncclAllReduce), with the R rank pointers of the simulated group passed as
 * arrays.  Two protocols from the page's MemoryChannel table are offered:
 *
 *   arProtoLL  low latency: one kernel, flag-carrying 8-byte packets (16-byte
 *              ones as an option), polled per wavefront; meant for
 *              decode-size messages.
 *   arProtoHB  high bandwidth: two-shot reduce-scatter by chunk then
 *              all-gather, 128-bit bulk loads and stores, no flags; meant for
 *              prefill-size messages.  A staged form with a kernel boundary
 *              between the shots is available as an option.
 *
 * Both give the same result: for every element i,
 *     a = x_0[i];  a = a + x_j[i] for j = 1..R-1 (binary32, in this order);
 *     recv_r[i] = a rounded to the element type (round to nearest even),
 * which is one reading of a SUM all-reduce over float/float16/bfloat16, the
 * operations and types admitted by the runtime guards of "SGLang 中的 MSCCL++
 * All-Reduce 基准测试与推理集成指南" (blog.gitcode.com), section 4.3.
 *
 * Errors are return codes; nothing here aborts, throws or prints (except with
 * the environment variable AR_DEBUG=1, which logs rejected calls to stderr).
 * A result of arUnsupported means "use another all-reduce", the fallback the
 * SGLang guide describes when a guard fails (sections 4.3 and 5).
 *
 * All entry points are host functions.  A communicator is used from one host
 * thread and one stream at a time, like an NCCL communicator: its LL packet
 * memory is shared by its calls, so two LL calls of one communicator must not
 * overlap in time.  Several communicators may run at once on different
 * streams.  An LL call needs all of its workgroups resident together, so
 * concurrent kernels that fill the GPU can delay an LL call up to its wait
 * bound (arOptPollTimeoutUs), after which it records arTimeout.
 */
#ifndef AR_ALLREDUCE_H
#define AR_ALLREDUCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AR_VERSION 10200 /* 1.2.0 */
#define AR_MAX_RANKS 32

typedef struct arComm *arComm_t;

/* A hipStream_t, passed as an untyped pointer so that this header does not
 * need the HIP headers.  NULL is the device's null stream. */
typedef void *arStream_t;

typedef enum {
    arSuccess = 0,
    arInvalidArgument = 1, /* a pointer, size, alignment or overlap rule broken */
    arUnsupported = 2,     /* valid request this library does not serve: fall back */
    arInvalidUsage = 3,    /* request exceeds what the communicator was made for */
    arHipError = 4,        /* a HIP runtime call failed */
    arTimeout = 5,         /* an LL packet wait ran out of time (asynchronous) */
    arInternalError = 6
} arResult_t;

typedef enum { arBfloat16 = 0, arFloat16 = 1, arFloat32 = 2 } arDataType_t;

typedef enum { arSum = 0 } arRedOp_t;

/* arProtoAuto picks, per message size, the protocol that arCommTune measured
 * faster (HB where nothing was tuned). */
typedef enum { arProtoLL = 0, arProtoHB = 1, arProtoAuto = 2 } arProtocol_t;

/* Tunables and test hooks, see arCommSetOption.  The launch-shape options
 * are the (workgroups, threads per workgroup) pairs that an auto-tuner would
 * time per message size. */
typedef enum {
    /* LL: longest total wait of one lane for packets, in microseconds
     * (default 2,000,000).  A wait that runs out records arTimeout in the
     * communicator and the kernel finishes without the missing data. */
    arOptPollTimeoutUs = 0,
    /* LL: workgroups per simulated rank; 0 = the built-in default for the
     * rank count and message size (a table measured on MI355X; with only
     * arOptLLThreads set, as many lanes per rank as the default has). */
    arOptLLBlocksPerRank = 1,
    /* HB: workgroups in the grid (rounded down to a multiple of nranks, at
     * least nranks, capped by the message's tiles); 0 = the built-in default:
     * one per compute unit, more from 4 MiB per rank for fewer than 6 ranks
     * (8 per CU at 1 rank down to 2 at 4 and 5) and for 9 to 15 ranks (2, or 4
     * above 16 MiB), where one per CU keeps too few loads in flight (measured
     * on MI355X); the default takes up to a quarter more workgroups where
     * that saves a workgroup a round of tiles (at most four rounds). */
    arOptHBBlocks = 2,
    /* HB: 1 = non-temporal loads and stores, 0 = ordinary (cached) ones.
     * -1 (default): the policy the tuner chose for the message size and mode,
     * else 1.  On MI355X ordinary accesses win from a few MiB per rank while
     * the message fits the last-level cache, non-temporal ones above it. */
    arOptHBNonTemporal = 3,
    /* Test hook: LL consumers wait for a flag shifted by this value, which no
     * producer writes when the value is not 0, so every wait times out.
     * Default 0. */
    arOptDebugFlagSkew = 4,
    /* HB: 16-byte vectors each lane handles per rank per step (1, 2 or 4;
     * capped at 2 above 4 ranks and at 1 above 8); 0 = default (1). */
    arOptHBUnroll = 5,
    /* LL: threads per workgroup (64, 128, 256, 512 or 1024; capped at 512
     * above 16 ranks); 0 = the built-in default for the rank count and
     * message size. */
    arOptLLThreads = 6,
    /* HB: threads per workgroup (64 .. 1024, a multiple of 64; capped at 512
     * above 8 ranks and 256 above 16); 0 = default (256 up to 8 ranks; 128
     * from 9 to 16 ranks up to 16 MiB per rank and 64 above; 128 from 17
     * ranks: the fastest measured on MI355X at the configured sizes). */
    arOptHBThreads = 7,
    /* HB: which elements simulated rank c reduces (its chunk) -- 0: the
     * contiguous c-th of R equal parts, 1: every R-th tile starting at tile c
     * (default; streams all R buffers in address order, which HBM serves
     * faster). */
    arOptHBChunkLayout = 8,
    /* Both protocols: hierarchical summation order for nodes of this many
     * consecutive ranks: each node's partial is summed in binary32 in rank
     * order, then the partials in node order, then rounded once -- the result
     * of a two-level all-reduce that reduces inside each node first and across
     * nodes second ("SGLang 中的 MSCCL++ All-Reduce 基准测试与推理集成指南",
     * section 4.4: multi-node algorithms for TP = 16 / 32).  0 (default), 1
     * or >= nranks: the flat order 0..R-1.  A value in between must divide
     * nranks (else arInvalidUsage).  The fused HB kernel and the LL kernel
     * fold the order in registers; with arOptHBStaged the HB call runs the
     * staged two-level form (see there).  The sequenced LL flag scheme keeps
     * the flat order: with it, LL returns arUnsupported (arProtoAuto then
     * runs HB). */
    arOptNodeRanks = 9,
    /* LL: packet width in bytes.  8: a 4-byte payload next to a 4-byte flag,
     * written as one 64-bit atomic store, so a reader that sees the flag also
     * sees the payload.  16: two such pairs, written and read as one 16-byte
     * access (half the memory instructions per payload byte); an ablation,
     * because it needs each 8-byte half of a 128-bit store to become visible
     * as a unit, which neither HIP (no 128-bit atomics) nor any gfx950
     * document guarantees.  0 (default) and 8: 8-byte packets; the tuner
     * times 8-byte packets only.  16 needs the communicator's packet memory
     * below 4 GiB (maxRanks * maxLLBytesPerRank * 2), else setting it returns
     * arUnsupported. */
    arOptLLPacketBytes = 10,
    /* HB: 1 = the staged two-shot, an ablation of the fused default: the
     * reduce-scatter writes each reduced chunk to its owner rank's output
     * only, a kernel boundary stands for the synchronisation between the
     * shots (the HB protocol synchronises rarely, "MSCCL++：让 GPU 通信像 CUDA
     * 一样可编程", "MemoryChannel"), and the all-gather copies each chunk from
     * its owner to the other outputs.  Same result bits; 2 * bytes per rank
     * more traffic and one more launch.  Launch shape from arOptHBThreads /
     * arOptHBBlocks or the defaults, never the tuned table.  0 (default): fused.
     *
     * With arOptNodeRanks = L set as well (R = G * L ranks in G nodes), the
     * staged two-level form of the same guide's section 4.4 multi-node
     * algorithms, and of the high-throughput mode of "NCCL EP统一MoE通信生态：
     * 打破碎片化，加速大模型推理新纪元" (itsolotime.com/archives/27456,
     * section 3.2: inside the node first, between nodes second): stage 1 is a
     * node-local reduce-scatter that writes each node's binary32 partial to
     * the communicator's workspace (arCommSetWorkspace: at least
     * G * roundup(count * 4, 256) bytes, else arInvalidUsage), a kernel
     * boundary separates the levels, and stage 2 folds the G partials of each
     * position in node order, rounds once and all-gathers the result to every
     * rank.  Same bits as the fused kernel in that order; 2 * G * count * 4
     * bytes more traffic.  Its default launch shape is 64 threads and four
     * workgroups per compute unit for both stages (measured fastest on
     * MI355X at 16 and 32 ranks); arOptHBThreads / arOptHBBlocks set it. */
    arOptHBStaged = 11,
    /* LL: how a packet left by an earlier call is kept from looking ready.
     * 0 (default): the reader zeroes every packet it has consumed, so packet
     * memory is zero between calls (one extra store per packet).  1: every
     * 512-byte group of a rank's packets carries a 32-bit sequence number in a
     * table owned by the communicator; producers flag packets with the
     * group's next number and the group's reader advances it, so nothing is
     * cleared.  An ablation: slower on MI355X at every LL size, since the
     * producer and the consumer of each group read its table entry before
     * they can store or poll (hardware counters show the two extra reads per
     * group), while the clears it saves are stores no one waits for.  Both
     * give the same results and may be mixed from call to call.  With 1, the launch shape
     * comes from the LL options or the defaults, never the tuned table. */
    arOptLLFlagScheme = 12,
    /* Test hook: the value arCommReset writes to every sequence-table entry
     * (0 .. 0xFFFFFFFF; default 0), to exercise the sequence numbers' wrap.
     * Takes effect at the next arCommReset. */
    arOptDebugSeqStart = 13,
    /* arCommTune's timing method.  0 (default): each candidate replays on
     * unchanged inputs, which stay in the last-level cache between calls, as
     * the benchmark's graph replays do.  1: before each timed call a copy-like
     * kernel rewrites the inputs (every 16-byte vector of each rank's
     * message), as when every step of a model produces new inputs; the
     * rewrites' own time, measured alone, is subtracted.  On MI355X this
     * changes the HB access policy that wins from a few MiB per rank up. */
    arOptTuneFreshInputs = 14,
    /* LL, bfloat16 and float16: the packet format.  1: three elements and a
     * 16-bit flag in each 8-byte packet (48 bits of payload, still one 64-bit
     * atomic store, so a reader that sees the flag sees the elements): a
     * third fewer packet and clear bytes than the word packet, whose
     * 4-byte payload sits next to a 4-byte flag.  0: the word packet.
     * -1 (default): three-element packets from the size where they measured
     * faster on MI355X (above 512 KiB per rank at 1, 2 and 4 ranks, 256 KiB
     * at 3 and 5 to 8, above 128 KiB from 9 to 16, 128 KiB above 16),
     * word packets below, where their LDS staging costs more than the bytes
     * they save.
     * Applies to the flat order, the cleared flag scheme and 8-byte packets;
     * float32, arOptNodeRanks, the sequenced scheme and 16-byte packets use
     * word packets.  A value other than -1 also turns the tuned LL entry off. */
    arOptLLDense = 15
} arOption_t;

/* The communicator is the long-lived group resource of an NCCL-style
 * collective library: it owns the buffers that every call reuses, so set-up
 * is paid once and each call only enqueues work (the group/handle split of
 * "NCCL EP统一MoE通信生态：打破碎片化，加速大模型推理新纪元",
 * itsolotime.com/archives/27456, section 2.3, 资源生命周期管理).  Its LL
 * packet memory must exist before a graph capture starts, because nothing can
 * be allocated inside one ("SGLang 中的 MSCCL++ All-Reduce 基准测试与推理集成指南",
 * blog.gitcode.com, section 1: the all-reduce runs under CUDA Graph decode).
 *
 * Create a communicator on `device` for groups of up to `maxRanks` (1..32)
 * simulated ranks and LL messages of up to `maxLLBytesPerRank` bytes per rank.
 * It owns device memory for the LL packets (2 * maxRanks * maxLLBytesPerRank
 * bytes, each rank's share rounded up to 512 bytes: packets are half payload,
 * half flags, at either width), a sequence table of 1/128 of that size (see
 * arOptLLFlagScheme) and a word that records an asynchronous error.  maxLLBytesPerRank
 * may be 0 (HB only).  Allocates with hipMalloc, so it must not be called
 * while a stream is being captured.  The caller's current device is left
 * unchanged.
 * Returns arInvalidArgument for a NULL `comm` or out-of-range sizes,
 * arHipError if the device or memory is not available. */
arResult_t arCommCreate(arComm_t *comm, int device, int maxRanks, size_t maxLLBytesPerRank);

/* Free the communicator and its device memory: the end of the long-lived
 * group resource (NCCL EP article, itsolotime.com/archives/27456, section
 * 2.3).  Work that uses it must have finished. */
arResult_t arCommDestroy(arComm_t comm);

/* Recovery of the group resource after a failed call, so the communicator
 * can be reused instead of rebuilt (NCCL EP article, section 2.3: the group's
 * buffers are long-lived and reused across calls).
 * Enqueue, on `stream`, a kernel that clears the LL packets, the sequence
 * table (to arOptDebugSeqStart, 0 by default) and the asynchronous error, so
 * that the communicator can be used again after a timeout (an LL call that
 * timed out may leave packets set; LL results are undefined until the reset).
 * No allocation and no memset node: safe to capture in a graph. */
arResult_t arCommReset(arComm_t comm, arStream_t stream);

/* Error reporting without aborts: the pages' integration never aborts on a
 * failed guard but reports it and falls back ("SGLang 中的 MSCCL++ All-Reduce
 * 基准测试与推理集成指南", sections 4.3 and 5); a device-side failure (an LL
 * wait that ran out) is kept in the communicator and read here.
 * Read the asynchronous error recorded by earlier kernels: arSuccess or
 * arTimeout.  Synchronises the device first.  The error stays set until
 * arCommReset. */
arResult_t arCommGetAsyncError(arComm_t comm, arResult_t *asyncError);

/* Device memory for the communicator's staged two-level HB form (arOptHBStaged
 * with arOptNodeRanks): the node partials that the node-local reduce-scatter
 * writes and the cross-node fold reads -- the scratch buffers that a
 * multi-node MSCCL++ algorithm exchanges between its levels ("SGLang 中的
 * MSCCL++ All-Reduce 基准测试与推理集成指南", section 4.4).  The caller owns
 * it: the library never allocates it, so it can come from the caller's
 * allocator and be set before a graph capture.  It must stay valid, and not
 * be used for anything else, while calls that use it are pending or captured.
 * `workspace` 256-byte aligned device memory of `bytes` bytes on the
 * communicator's device; NULL with 0 detaches it.  No HIP call.
 * Returns arInvalidArgument for a NULL comm, a pointer without a size (or the
 * reverse), or a misaligned pointer.  A call that needs more than `bytes`
 * returns arInvalidUsage, and one whose rank buffers overlap the part it
 * needs arInvalidArgument. */
arResult_t arCommSetWorkspace(arComm_t comm, void *workspace, size_t bytes);

/* Set or read one option (arOption_t) of the communicator: the per-size
 * launch parameters (workgroups, threads per workgroup) that SGLang's MSCCL++
 * integration times and keeps ("SGLang 中的 MSCCL++ All-Reduce 基准测试与推理
 * 集成指南", section 4.4), the protocol details of the MemoryChannel table's
 * LL and HB protocols ("MSCCL++：让 GPU 通信像 CUDA 一样可编程",
 * infinitensor.com/news/50, "MemoryChannel"), the two-level order of that
 * guide's section 4.4 multi-node algorithms, and test hooks.  Values outside
 * an option's range give arInvalidArgument. */
arResult_t arCommSetOption(arComm_t comm, arOption_t option, int64_t value);
arResult_t arCommGetOption(arComm_t comm, arOption_t option, int64_t *value);

/* Measure launch shapes and keep the fastest, per message size -- the
 * start-up tuning of SGLang's MSCCL++ integration ("SGLang 中的 MSCCL++
 * All-Reduce 基准测试与推理集成指南", blog.gitcode.com, section 4.4: every
 * power-of-two size timed over (workgroups, threads per workgroup) candidates,
 * the best kept for the life of the process).
 *
 * For `dtype` and `nranks`, every power-of-two size from 512 bytes up to
 * maxBytesPerRank per rank (the last bucket at maxBytesPerRank itself) is
 * timed with each protocol the communicator can run at that size, in place
 * and out of place (the two favour different shapes), over the built-in
 * default shape and a grid of candidates around it (HB: half, once and twice
 * the default workgroup count); a candidate wins only if it is
 * more than 3 % faster than the best before it, a winner other than the
 * default shape and access policy is timed again beside the default and kept
 * only if it is still more than 3 % faster (else the default is stored), and
 * the stored shape and its time are kept in the communicator.  Later calls of that dtype and rank count
 * use the stored shape of their size bucket (the message size rounded up to a
 * power of two) and mode (in place: recvbufs[r] == sendbufs[r] for every
 * rank) unless arOptLLThreads/arOptLLBlocksPerRank (LL) or arOptHBThreads/
 * arOptHBBlocks (HB), arOptLLPacketBytes or arOptLLFlagScheme are set;
 * arProtoAuto then picks the faster protocol.  LL candidates use 8-byte
 * packets in the default flag scheme; HB candidates both access policies
 * unless arOptHBNonTemporal fixes one.
 * Tuning again overwrites the table; sizes never tuned use built-in defaults.
 *
 * Each candidate is timed the way latency-sensitive callers run the library:
 * its calls captured into a HIP graph on a private stream of the tuner, and
 * the graph replayed (eager launches would time the host's launch rate at
 * small sizes); with arOptTuneFreshInputs = 1, each call right after a
 * rewrite of its inputs, the rewrites' time subtracted.  Allocates two scratch planes of nranks * maxBytesPerRank
 * bytes for the duration, waits for `stream` first and synchronises the
 * device at the end: never call it while a stream is being captured.
 * Returns arInvalidArgument for a NULL comm or maxBytesPerRank outside
 * 512 B .. 16 GiB, arUnsupported for a dtype or rank
 * count arAllReduce would reject, arInvalidUsage if the communicator is not on
 * the current device, arHipError if memory or a launch fails, arTimeout if an
 * LL wait ran out during tuning (then reset the communicator). */
arResult_t arCommTune(arComm_t comm, arDataType_t dtype, int nranks, size_t maxBytesPerRank,
                      arStream_t stream);

/* One entry of the tuned table (the guide's best_configs entry for one size,
 * section 4.4). */
typedef struct {
    int tuned;        /* 0: this size was never tuned (the rest is 0) */
    int threads;      /* threads per workgroup that won; 0 with blocks 0: the default shape */
    int blocks;       /* workgroups that won (HB: the grid; LL: per rank) */
    int packetBytes;  /* LL: the packet width it was timed with (8); HB: 0 */
    int nonTemporal;  /* HB: 1 if non-temporal accesses won, 0 if cached ones; LL: 0 */
    float us;         /* time per call measured for it, in microseconds */
} arTunedShape_t;

/* Look-up of the tuned table as the guide's section 4.4 describes it: the
 * message size rounded up to a power of two selects the entry.
 * The tuned entry for (dtype, nranks, protocol LL or HB) at a message of
 * bytesPerRank bytes, in place (inPlace = 1) or out of place (inPlace = 0),
 * copied to *shape.  Returns arInvalidArgument for NULL pointers or
 * out-of-range arguments. */
arResult_t arCommGetTunedShape(arComm_t comm, arDataType_t dtype, int nranks,
                               arProtocol_t protocol, size_t bytesPerRank, int inPlace,
                               arTunedShape_t *shape);

/* The launch behind the communicator's most recent call (arAllReduce, or a
 * tuning candidate of arCommTune): the (workgroups, threads per workgroup)
 * pair that SGLang's tuner picks per size ("SGLang 中的 MSCCL++ All-Reduce
 * 基准测试与推理集成指南", section 4.4), with the protocol details that go
 * with it, so that a caller or a profile can name the shape a timed call ran.
 * protocol is -1 before the first launch; a call that enqueued nothing
 * (count 0, or an error) leaves the record as it was. */
typedef struct {
    int protocol;      /* arProtoLL or arProtoHB (arProtoAuto resolved); -1: none yet */
    int kernels;       /* kernels the call enqueued (2 for a staged HB form) */
    unsigned grid;     /* workgroups of its (first) kernel */
    unsigned threads;  /* threads per workgroup */
    int packetBytes;   /* LL: packet width, 8 or 16; HB: 0 */
    int nonTemporal;   /* HB: 1 non-temporal accesses, 0 cached; LL: 0 */
    int nodeRanks;     /* ranks per node of a hierarchical order; 0: flat */
    int staged;        /* HB: 1 for a staged form; else 0 */
    int packetPayloadBytes; /* LL: payload bytes per packet -- 4 (8-byte word packet),
                             * 6 (three 16-bit elements), 8 (16-byte packet); HB: 0 */
} arLaunchInfo_t;

/* Copy the record of the most recent launch to *info.  Returns
 * arInvalidArgument for NULL pointers. */
arResult_t arCommGetLastLaunch(arComm_t comm, arLaunchInfo_t *info);

/* The sum all-reduce.
 *
 *  sendbufs  host array of `nranks` device pointers; sendbufs[r] holds rank
 *            r's `count` elements, contiguous.  Read only during the call.
 *  recvbufs  host array of `nranks` device pointers for the results, laid
 *            out like sendbufs.  recvbufs[r] == sendbufs[r] for a rank means
 *            in place; the result is then computed from the values the
 *            buffers held when the kernel started.
 *  count     elements per rank.  0 returns arSuccess and enqueues nothing.
 *  dtype     arBfloat16, arFloat16 or arFloat32 (else arUnsupported).
 *  op        arSum only (else arUnsupported).
 *  nranks    1..32 (else arUnsupported); 1 is a copy.
 *  protocol  arProtoLL, arProtoHB or arProtoAuto (else arInvalidArgument).
 *  comm      a communicator on the current device.
 *  stream    the stream to enqueue on.
 *
 * Rules (arInvalidArgument when broken): no NULL pointer; every pointer
 * 16-byte aligned; the 2*nranks byte ranges do not overlap except that a
 * receive buffer may coincide exactly with the same rank's send buffer, and
 * send buffers may overlap one another (they are only read).
 * LL also needs nranks <= the communicator's maxRanks and count * element
 * size <= its maxLLBytesPerRank (arInvalidUsage otherwise); arProtoAuto only
 * picks LL where it can run.  With a hierarchical order set (arOptNodeRanks),
 * nranks must be a multiple of the node size (arInvalidUsage otherwise), and
 * the staged HB form and the sequenced LL scheme return arUnsupported.
 *
 * The call only enqueues work and returns; the buffers belong to the caller
 * and must stay valid until the work has run (for a captured graph, as long
 * as the graph is replayed).  Nothing is allocated or synchronised, so calls
 * can be captured into a HIP graph.  Validation makes no HIP call, so every
 * argument error is reported without touching the device. */
arResult_t arAllReduce(const void *const *sendbufs, void *const *recvbufs, size_t count,
                       arDataType_t dtype, arRedOp_t op, int nranks, arProtocol_t protocol,
                       arComm_t comm, arStream_t stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc -- and so
 * cannot create a communicator: the HB all-reduce with no communicator and
 * no allocation of any kind.
 *
 * nodeRanks 0, 1 or >= nranks: the fused HB two-shot in the flat order
 * 0..R-1 (no scratch).  1 < nodeRanks < nranks: the staged two-level form
 * of arOptHBStaged with arOptNodeRanks = nodeRanks (node partials, a kernel
 * boundary, the fold across nodes), same bits as arAllReduce there, with
 * the node partials in a scratch array that the library holds in device
 * memory, one per GPU it runs on, for the life of the process:
 * AR_NOALLOC_SCRATCH_BYTES (64 MiB), so (nranks / nodeRanks) *
 * roundup(count * 4, 256) bytes must fit (else arInvalidUsage; larger
 * messages take arAllReduce with a workspace).  Nothing in the scratch needs
 * to start at any value: every call writes the partials it reads.
 *
 * Runs on the current device with arAllReduce's default launch shapes for
 * the form it takes (no options), non-temporal accesses, interleaved chunks.
 * The arguments and their rules are arAllReduce's (protocol HB); nodeRanks
 * outside 0..32 is arInvalidArgument, a nodeRanks in between that does not
 * divide nranks arInvalidUsage.  The first call on a device looks up the
 * scratch's address and the device's compute units (no allocation).
 * All calls on one GPU share its scratch, which keeps the last call's
 * contents: two two-level calls that overlap in time on one GPU (on streams
 * with no ordering between them) race, and their results are undefined.
 * Calls on one stream, or captured into one graph, are ordered and safe. */
#define AR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
arResult_t arAllReduceNoAlloc(const void *const *sendbufs, void *const *recvbufs, size_t count,
                              arDataType_t dtype, arRedOp_t op, int nranks, int nodeRanks,
                              arStream_t stream);

/* Static description of a result code (arUnsupported is the guide's
 * "fall back to another all-reduce", sections 4.3 and 5). */
const char *arGetErrorString(arResult_t result);

/* AR_VERSION of the built library, so a caller can check the ABI it loaded
 * (the NCCL-compatible API of "MSCCL++：让 GPU 通信像 CUDA 一样可编程",
 * "第一层：Collective API", is a drop-in replacement and needs one). */
int arGetVersion(void);

#ifdef __cplusplus
}
#endif

#endif /* AR_ALLREDUCE_H */
