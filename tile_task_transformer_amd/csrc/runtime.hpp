// Tiled tensors and the sequential-task-flow executor (internal C++ API).
//
// The executor implements the runtime side of the method described in the
// pith.science review of NNTile ("What carries the argument"): tasks are
// submitted in program order, each names the tiles it reads and writes, and
// the ordering between tasks is inferred from those accesses alone:
//   read  after write  (RAW): a reader waits for the tile's last writer;
//   write after read   (WAR): a writer waits for every reader since then;
//   write after write  (WAW): a writer waits for the previous writer.
// Ready tasks are mapped onto a small set of HIP streams (one GPU); an edge
// between tasks on the same stream is free (streams are FIFO), an edge that
// crosses streams becomes an event record + hipStreamWaitEvent.
#pragma once

#include <chrono>
#include <functional>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "common.hpp"

struct tt_ctx;

namespace tt {

struct TileState {
  int64_t last_writer = -1;        // task id of the last writer
  std::vector<int64_t> readers;    // task ids that read since that write
};

// Residency of one tile whose home is pinned host memory.
struct Residency {
  float* dev = nullptr;            // device copy in the context's arena (null if not resident)
  size_t off = 0, bytes = 0;       // its arena offset and size
  bool dev_valid = false;          // device copy holds the latest value
  bool host_valid = true;          // host copy holds the latest value
  int64_t last_use = -1;           // id of the last task that used it (LRU order)
  int64_t need = -1;               // id of the latest task being launched that accesses it
  int64_t protect = -1;            // prefetched for tasks with id <= protect (evicted only under pressure)
  std::vector<int64_t> users;      // launched tasks that touched the device copy since its last launched writer
  std::vector<int64_t> future;     // ids of the tasks in the launching window that access it (ascending)
  size_t fpos = 0;                 // first entry of `future` not yet passed
  int wb_event = -1;               // event after its last write-back (host copy in flight until then)
  int ready_event = -1;            // copy-stream event after which the device copy is usable (-1: already)
  bool staged = false;             // in tt_ctx::staged (awaiting its ready event)
};

}  // namespace tt

struct tt_tensor {
  tt_ctx* ctx = nullptr;
  int64_t id = 0;
  int ndim = 0;
  int64_t shape[TT_MAX_DIMS] = {};
  int64_t tshape[TT_MAX_DIMS] = {};
  int64_t grid[TT_MAX_DIMS] = {};
  int dtype = TT_F32;
  int home = TT_HOME_DEVICE;
  int mat_split = 1;               // leading dims that form the rows of a tile's matrix view
  int64_t ntiles = 0;
  int64_t elems = 0;
  std::vector<int64_t> tile_off;   // element offset of each tile (tile-major)
  std::vector<tt::TileState> state;
  char* base = nullptr;            // device base (device home)
  char* host = nullptr;            // pinned host base (pinned home)
  bool owned = false;
  std::vector<tt::Residency> res;  // pinned home only
  std::string name;

  size_t esize() const { return 4; }
  int64_t bytes() const { return elems * (int64_t)esize(); }
  // extents of tile `lin`
  void extent(int64_t lin, int64_t* ext) const;
  int64_t tile_elems(int64_t lin) const;
  int64_t lin(const int64_t* idx) const;
  // rows/cols of the matrix view of tile `lin`
  void mat(int64_t lin, int64_t* rows, int64_t* cols) const;
  // device pointer of tile `lin` (valid at launch time; residency handled by the executor)
  void* dev(int64_t lin) const;
};

namespace tt {

struct TileRef {
  tt_tensor* t = nullptr;
  int64_t lin = -1;
  bool valid() const { return t != nullptr; }
};

struct Access {
  TileRef ref;
  int mode;  // TT_R, TT_W, TT_RW
};

using LaunchFn = std::function<int(hipStream_t stream, void* workspace)>;

struct Task {
  int64_t id = 0;
  char label[32] = {};
  std::vector<int64_t> deps;
  std::vector<Access> acc;
  LaunchFn run;
  double cost = 0.0;  // flop estimate (0 = unknown, treated as light)
  int stream = -1;
  bool need_event = false;
};

struct Launched {
  int stream = -1;
  int64_t seq = -1;        // position on its stream (1-based)
  int event = -1;          // index into the event pool, -1 = none recorded
};

struct TaskRecord {        // kept for tt_dump_dag
  int64_t id;
  std::string label;
  int stream;
  std::vector<int64_t> deps;
  std::vector<std::pair<int64_t, std::pair<int64_t, int>>> acc;  // tensor id, tile lin, mode
  double cost = 0.0;       // flop estimate (0 for memory-bound tasks)
};

}  // namespace tt

struct tt_ctx {
  int device = 0;
  bool dryrun = false;
  int n_streams = 1;
  int active_streams = 1;  // tasks go to streams 0..active_streams-1
  double heavy_flops = 0;  // > 0: tasks of at least this cost run in order on stream 0
  bool priorities = false;  // launch each window by critical-path priority (device homes only)
  int window = 512;
  size_t budget = 0;
  bool record = false;
  int latched = TT_OK;             // first asynchronous/launch error
  std::string latched_msg;

  std::vector<hipStream_t> streams;
  bool owns_streams = true;            // false: borrowed from the caller (tt_ctx_create_on_streams)
  hipStream_t copy_stream = nullptr;   // residency H2D
  hipStream_t d2h_stream = nullptr;    // residency write-backs (the link is full duplex)
  std::vector<void*> workspace;        // per stream
  size_t workspace_bytes = 0;

  // task ids
  int64_t next_id = 0;
  int64_t done_below = 0;              // tasks with id < done_below are complete
  int64_t window_base = 0;             // id of pending[0]
  std::vector<tt::Task> pending;
  std::vector<tt::Launched> launched;  // index id - launched_base
  int64_t launched_base = 0;

  // per-stream bookkeeping
  std::vector<int64_t> stream_seq;     // tasks launched on each stream
  std::vector<int64_t> last_assigned;  // id of the last task assigned to each stream
  std::vector<std::vector<int64_t>> waited;  // waited[s][t] = highest seq of t waited by s
  int rr = 0;

  // events
  std::vector<hipEvent_t> events;
  int events_used = 0;
  std::vector<hipEvent_t> ext_events;  // tt_ctx_wait_stream / tt_ctx_join_stream
  int ext_events_init();

  // residency of pinned-host tiles: device copies live in one arena of
  // `budget` bytes (first-fit with coalescing); LRU eviction writes dirty
  // tiles back on the copy stream
  char* arena = nullptr;
  size_t arena_bytes = 0;
  std::map<size_t, size_t> arena_free;  // offset -> size
  std::vector<tt::TileRef> resident;    // tiles with a device copy
  int64_t cur_task = -1;                // id of the task being launched
  // copy-stream ordering of staged tiles: each tile gets the event recorded
  // right after its own staging (its range freed of earlier occupants, its
  // data copied in), so a task waits for its own tiles and not for the
  // prefetches of later tasks queued behind them
  std::vector<tt::Residency*> staged;   // staged since the last ready event
  std::vector<int> ready_seq;           // per event index: its position among ready events (ascending)
  int ready_count = 0;                  // ready events recorded since the last drain
  std::vector<int> waited_copy;         // per stream: highest ready position it waited on
  int mark_ready();
  int arena_init();
  int arena_alloc(size_t bytes, size_t* off, bool soft, int64_t use);
  void arena_release(size_t off, size_t bytes);
  int evict_one(bool spare_prefetched, int64_t use);
  int64_t next_use(tt::Residency& r);
  // arena ranges freed by a write-back still in flight: (offset, bytes, event)
  struct DirtyFree {
    size_t off, bytes;
    int event;
  };
  std::vector<DirtyFree> dirty_free;
  std::vector<tt::Residency*> planned;  // tiles whose `future` this window filled
  int wait_dirty_free(size_t off, size_t bytes, hipStream_t s);
  int wait_users(tt_tensor* t, int64_t lin, hipStream_t s);
  int prefetch(size_t i);
  int clean_ahead(size_t i);
  void plan_window();
  void unplan_window();
  void drop_resident(tt_tensor* t);

  // per-task GPU timing (tt_ctx_profile): event pairs around matching launches
  bool prof_on = false;
  std::string prof_filter;             // "*" = every task
  int prof_every = 1;                  // time every n-th matching task
  int64_t prof_seen = 0;               // matching tasks since tt_ctx_profile
  struct ProfRec {
    std::string label;
    int ev0, ev1;
  };
  std::vector<ProfRec> prof_pending;
  std::vector<hipEvent_t> prof_events;
  int prof_used = 0;
  hipEvent_t prof_base = nullptr;      // recorded by tt_ctx_profile on an idle device
  bool prof_base_set = false;
  std::vector<std::pair<float, float>> prof_iv;  // [start, end] of each timed task, ms after prof_base
  struct ProfAgg {
    int64_t count = 0;
    double total = 0, mn = 1e30, mx = 0;
  };
  std::vector<std::pair<std::string, ProfAgg>> prof_agg;
  int prof_collect();

  int64_t next_tensor_id = 0;
  std::vector<tt_tensor*> tensors;     // live tensors
  int has_pinned = 0;                  // live tensors whose home is pinned host
  std::vector<tt::TaskRecord> records;
  tt_stats stats = {};

  // ---- internal API
  int submit(const char* label, std::vector<tt::Access> acc, tt::LaunchFn run, double cost = 0.0);
  int flush();
  int flush_window();  // flush's body: assign streams, add events, launch the pending window
  std::vector<size_t> launch_order();  // positions in `pending`, in the order they are launched
  int wait_all();
  void forget_launched();  // bookkeeping after a drain: nothing submitted so far is pending

  // graph capture: the tasks submitted between capture_begin and capture_end
  // are recorded (not run) into one executable graph, replayed with
  // graph_launch
  bool capturing = false;
  int64_t workspace_gen = 0;  // bumped when the per-stream workspaces move (recorded graphs go stale)
  int capture_begin();
  int capture_end(hipGraphExec_t* out);  // out may be null (discard)
  int graph_launch(hipGraphExec_t exec);
  int ensure_workspace(size_t bytes);
  tt::Launched* info(int64_t id);
  int acquire_event(int* idx);
  int make_resident(tt::Task& task, hipStream_t s);
};

namespace tt {
int tensor_create(tt_ctx* ctx, int ndim, const int64_t* shape, const int64_t* tshape, int dtype,
                  int home, int mat_split, const char* name, tt_tensor** out);
inline Access R(tt_tensor* t, int64_t lin) { return Access{TileRef{t, lin}, TT_R}; }
inline Access W(tt_tensor* t, int64_t lin) { return Access{TileRef{t, lin}, TT_W}; }
inline Access RW(tt_tensor* t, int64_t lin) { return Access{TileRef{t, lin}, TT_RW}; }
}  // namespace tt
