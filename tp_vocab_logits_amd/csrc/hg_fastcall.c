/*
 * _hgcall: fast-call Python wrappers of the per-call entry points of
 * libhg.so (hg_gather, hg_push, hg_collect, hg_stock_gather), for loops where
 * the ctypes conversion of the arguments (about 0.5 us a call) is a sizeable
 * part of a 3 us M=1 gather.
 * Argument marshalling only: every argument is an integer (a handle, a
 * host-array address, a row count, a device address, a stream), passed on
 * unchanged; the return value is the library's status code.
 *
 * The module does not link against libhg.so: bind() receives the addresses of
 * the four entry points from the already loaded library (see _lib.fast()).
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>

typedef int (*gather_fn)(void *h, const void *const *shards, int m, void *out, void *stream);
typedef int (*push_fn)(void *h, const void *const *shards, int m, void *stream);
typedef int (*collect_fn)(void *h, int m, void *out, void *stream);
typedef int (*stock_fn)(int tp, int shard, const void *const *shards, int m, void *out,
                        int vocab, void *stream);

static gather_fn g_gather;
static push_fn g_push;
static collect_fn g_collect;
static stock_fn g_stock;

static int as_ptr(PyObject *o, void **p) {
  *p = PyLong_AsVoidPtr(o);
  return !(*p == NULL && PyErr_Occurred());
}

static int as_int(PyObject *o, int *v) {
  long x = PyLong_AsLong(o);
  if (x == -1 && PyErr_Occurred()) return 0;
  if (x < INT_MIN || x > INT_MAX) {
    PyErr_SetString(PyExc_OverflowError, "integer argument out of range");
    return 0;
  }
  *v = (int)x;
  return 1;
}

static int check_bound(void *fn, Py_ssize_t nargs, Py_ssize_t want) {
  if (!fn) {
    PyErr_SetString(PyExc_RuntimeError, "_hgcall: bind() has not been called");
    return 0;
  }
  if (nargs != want) {
    PyErr_Format(PyExc_TypeError, "expected %zd arguments, got %zd", want, nargs);
    return 0;
  }
  return 1;
}

/* bind(gather_addr, push_addr, collect_addr, stock_addr) */
static PyObject *py_bind(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
  void *a, *b, *c, *d;
  (void)self;
  if (nargs != 4) {
    PyErr_SetString(PyExc_TypeError, "bind expects four function addresses");
    return NULL;
  }
  if (!as_ptr(args[0], &a) || !as_ptr(args[1], &b) || !as_ptr(args[2], &c) ||
      !as_ptr(args[3], &d))
    return NULL;
  if (!a || !b || !c || !d) {
    PyErr_SetString(PyExc_ValueError, "bind: null function address");
    return NULL;
  }
  g_gather = (gather_fn)a;
  g_push = (push_fn)b;
  g_collect = (collect_fn)c;
  g_stock = (stock_fn)d;
  Py_RETURN_NONE;
}

/* gather(handle, shards_array_addr, m, out_addr, stream) -> status */
static PyObject *py_gather(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
  void *h, *shards, *out, *stream;
  int m;
  (void)self;
  if (!check_bound((void *)g_gather, nargs, 5)) return NULL;
  if (!as_ptr(args[0], &h) || !as_ptr(args[1], &shards) || !as_int(args[2], &m) ||
      !as_ptr(args[3], &out) || !as_ptr(args[4], &stream))
    return NULL;
  return PyLong_FromLong(g_gather(h, (const void *const *)shards, m, out, stream));
}

/* push(handle, shards_array_addr, m, stream) -> status */
static PyObject *py_push(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
  void *h, *shards, *stream;
  int m;
  (void)self;
  if (!check_bound((void *)g_push, nargs, 4)) return NULL;
  if (!as_ptr(args[0], &h) || !as_ptr(args[1], &shards) || !as_int(args[2], &m) ||
      !as_ptr(args[3], &stream))
    return NULL;
  return PyLong_FromLong(g_push(h, (const void *const *)shards, m, stream));
}

/* collect(handle, m, out_addr, stream) -> status */
static PyObject *py_collect(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
  void *h, *out, *stream;
  int m;
  (void)self;
  if (!check_bound((void *)g_collect, nargs, 4)) return NULL;
  if (!as_ptr(args[0], &h) || !as_int(args[1], &m) || !as_ptr(args[2], &out) ||
      !as_ptr(args[3], &stream))
    return NULL;
  return PyLong_FromLong(g_collect(h, m, out, stream));
}

/* stock(tp, shard, shards_array_addr, m, out_addr, vocab, stream) -> status */
static PyObject *py_stock(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
  void *shards, *out, *stream;
  int tp, shard, m, vocab;
  (void)self;
  if (!check_bound((void *)g_stock, nargs, 7)) return NULL;
  if (!as_int(args[0], &tp) || !as_int(args[1], &shard) || !as_ptr(args[2], &shards) ||
      !as_int(args[3], &m) || !as_ptr(args[4], &out) || !as_int(args[5], &vocab) ||
      !as_ptr(args[6], &stream))
    return NULL;
  return PyLong_FromLong(g_stock(tp, shard, (const void *const *)shards, m, out, vocab, stream));
}

static PyMethodDef methods[] = {
    {"bind", (PyCFunction)(void (*)(void))py_bind, METH_FASTCALL,
     "bind(gather, push, collect, stock)"},
    {"gather", (PyCFunction)(void (*)(void))py_gather, METH_FASTCALL,
     "gather(handle, shards_addr, m, out_addr, stream) -> status"},
    {"push", (PyCFunction)(void (*)(void))py_push, METH_FASTCALL,
     "push(handle, shards_addr, m, stream) -> status"},
    {"collect", (PyCFunction)(void (*)(void))py_collect, METH_FASTCALL,
     "collect(handle, m, out_addr, stream) -> status"},
    {"stock", (PyCFunction)(void (*)(void))py_stock, METH_FASTCALL,
     "stock(tp, shard, shards_addr, m, out_addr, vocab, stream) -> status"},
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_hgcall",
                                    "Fast-call wrappers of libhg.so's per-call entry points.",
                                    -1, methods};

PyMODINIT_FUNC PyInit__hgcall(void) { return PyModule_Create(&module); }
